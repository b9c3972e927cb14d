// C ABI of libkvq (declared in include/kvq.h): host-side validation, workspace sizing, the
// split-count heuristic, launches on the caller's stream, and the checked (syncing) mode.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <unordered_set>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"
#include "kvq_layout.h"

namespace {

constexpr int kMaxSplits = 4096;
constexpr int kMaxGqa = 16;

constexpr int32_t kMaxKvHeads = 65535;

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_cache(const kvq_cache_t *c) {
  if (!c) return KVQ_ERR_INVALID_ARG;
  if (c->dtype != KVQ_INT8_Q8_0 && c->dtype != KVQ_BF16 && c->dtype != KVQ_INT8_PER_HEAD) return KVQ_ERR_UNSUPPORTED;
  if (c->block_size != kvq::kPage) return KVQ_ERR_UNSUPPORTED;
  if (c->head_dim != 128 && c->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return KVQ_ERR_INVALID_ARG;
  if (c->num_kv_heads > kMaxKvHeads) return KVQ_ERR_UNSUPPORTED;  // the writers' grid has a row per KV head
  if ((int64_t)c->num_blocks * kvq::kPage > INT32_MAX) return KVQ_ERR_INVALID_ARG;
  if (!c->k || !c->v || !aligned(c->k, 256) || !aligned(c->v, 256)) return KVQ_ERR_INVALID_ARG;
  if (c->dtype != KVQ_BF16) {
    if (!c->k_scales || !c->v_scales || !aligned(c->k_scales, 256) || !aligned(c->v_scales, 256))
      return KVQ_ERR_INVALID_ARG;
  }
  return KVQ_OK;
}

int check_heads(const kvq_cache_t *c, int32_t num_q_heads) {
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
  if (num_q_heads / c->num_kv_heads > kMaxGqa) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Several query tokens: a workgroup holds up to 64 (query token, head) rows, 4 tiles of 16; longer
// runs of query tokens (a prefill chunk) are cut into chunks of qchunk tokens, each attending over
// the keys up to its own last token.
int qchunk_for(int nq, int G) { return nq <= 64 / G ? nq : 64 / G; }
int chunks_for(int nq, int G) { return (nq + qchunk_for(nq, G) - 1) / qchunk_for(nq, G); }
int row_tiles_for(int nq, int G) { return nq > 1 ? (qchunk_for(nq, G) * G + 15) / 16 : 1; }
// Row tiles per workgroup: the waves of one workgroup share its pages across up to 4 tiles.
int rtw_for(int row_tiles) { return row_tiles >= 3 ? 4 : row_tiles; }

// Split count: enough workgroups to fill every compute unit, but no split shorter than a
// minimum number of pages, so that the merge stays small next to the stream.  A single sequence
// runs best with one workgroup (one wave per SIMD) per compute unit and long page runs per wave.
// A batch gets two workgroups per compute unit: its sequences' lengths differ, and the second
// workgroup per CU evens out the longest ones (the host sees only the maximum length).  A batch
// with fewer (sequence, KV head) pairs than compute units gets four: every split is cpp =
// max_pages / NS pages long, so a sequence shorter than the maximum fills only its share of its
// NS splits (the rest exit at once), and with few pairs the longest sequence's splits are the
// critical path.  These choices come from split-count sweeps of the INT8 and BF16 kernels on 256
// CUs: one sequence at 4K and 32K tokens; 32 sequences of 512-8K (best at 2); 4 sequences of
// 2K/8K/16K/32K (best at 128, 6% slower at this rule's 64) and 4 of 32K (best at 64, 14% slower
// at 128).  Which of the last two a batch is takes its lengths: choose_splits_lengths.
// Several query tokens per sequence (row_tiles > 1): a workgroup holds rtw 16-row tiles of
// (query token, head) pairs, and the count is set by the workgroups per (sequence, KV head), as
// for one query token.  Workgroups of 4 tiles (one wave per tile) keep no merge scratch in LDS,
// so two fit on a CU and count as two slots (three for q8_0 prompt sections, whose kernel keeps
// its registers within 3 waves per SIMD).  A q8_0 single chunk of 3 or 4 tiles runs as one
// 8-wave workgroup per CU (two page groups), one slot.  Prompt sections (several query chunks)
// get at least four rounds of workgroups, so that the last, partly filled round is short.
// Sweeps at 32K: 8 query tokens run best at 64 splits of the two-group form (48 and 96 are 19%
// and 45% slower); a 2048-token section takes 6.3 ms at 1 split, 5.5 ms at 2 and 5.1 ms at 4
// (this rule gives 3).
int choose_splits(int dtype, int S, int Hkv, int D, int max_context_len, int cus, int row_tiles = 1,
                  int chunks = 1) {
  (void)D;
  const int64_t max_pages = ((int64_t)max_context_len + kvq::kPage - 1) / kvq::kPage;  // (64-bit: no overflow)
  if (max_pages <= 0) return 1;
  const int rtw = rtw_for(row_tiles), groups = (row_tiles + rtw - 1) / rtw * chunks;
  // workgroups resident at once: 4-tile workgroups fit two per CU, three for q8_0 prompt sections
  // (their kernel is capped at 3 waves' registers per SIMD); a q8_0 single chunk's 8-wave
  // workgroup fills a CU
  const int per_cu = (row_tiles > 1 && rtw == 4) ? (dtype == KVQ_INT8_Q8_0 ? (chunks > 1 ? 3 : 1) : 2) : 1;
  const int64_t slots = (int64_t)per_cu * cus;
  const int64_t base = (int64_t)S * Hkv * groups;
  int64_t target_wg = ((int64_t)S * groups > 1 ? 2LL : 1LL) * slots;
  if (row_tiles == 1 && S > 1 && (int64_t)S * Hkv < cus) target_wg = 4 * slots;  // few pairs
  if (chunks > 1 && target_wg < 4 * slots) target_wg = 4 * slots;
  int64_t ns = (target_wg + base - 1) / base;
  const int min_pages = 8;
  const int64_t cap = (max_pages + min_pages - 1) / min_pages;
  if (ns > cap) ns = cap;
  if (ns < 1) ns = 1;
  if (ns > kMaxSplits) ns = kMaxSplits;
  return (int)ns;
}

// Split count from the batch's actual lengths (host copy).  One sequence, or at least as many
// (sequence, KV head) pairs as compute units: as choose_splits.  Fewer pairs: the split length
// cpp is set so that the non-empty workgroups (sequence s fills ceil(P_s / cpp) splits per KV
// head) make about four rounds of the compute units, no split shorter than 8 pages, a multiple
// of 4 pages; NS is then what the longest sequence needs.  Sweeps on 256 CUs: 4 sequences of
// 2K/8K/16K/32K tokens get 128 splits (the best measured; 137, from 15-page splits, was 3%
// slower), 4 of 32K get 64 (best).
int choose_splits_lengths(int dtype, int S, int Hkv, int D, const int32_t *lens, int cus) {
  int64_t total = 0;
  int max_len = 0;
  for (int s = 0; s < S; ++s) {
    total += ((int64_t)lens[s] + kvq::kPage - 1) / kvq::kPage;  // (64-bit: no overflow near INT32_MAX)
    max_len = std::max(max_len, (int)lens[s]);
  }
  if (max_len <= 0) return 1;
  if (S == 1 || (int64_t)S * Hkv >= cus) return choose_splits(dtype, S, Hkv, D, max_len, cus);
  const int min_pages = 8;
  const int64_t target = 4LL * cus;
  // (rounded up to a multiple of 4 pages: a split's pages are dealt to the workgroup's 4 waves)
  const int64_t cpp = (std::max<int64_t>(min_pages, (total * Hkv + target - 1) / target) + 3) / 4 * 4;
  const int64_t max_pages = ((int64_t)max_len + kvq::kPage - 1) / kvq::kPage;
  const int64_t ns = std::min<int64_t>(std::max<int64_t>(1, (max_pages + cpp - 1) / cpp), kMaxSplits);
  return (int)ns;
}

size_t workspace_bytes(int S, int Hq, int NS, int D) {
  const size_t rows = (size_t)S * Hq * NS;
  size_t o = rows * D * sizeof(float);
  o = (o + 255) & ~(size_t)255;
  return o + rows * 2 * sizeof(float);
}

int waves_for(int dtype, int D) {
  (void)dtype;
  (void)D;
  return 4;
}

bool is_capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return false;
  return cs != hipStreamCaptureStatusNone;
}

bool bf16_finite(uint16_t b) { return (b & 0x7F80u) != 0x7F80u; }

// Validates the decode arguments and fills the kernel argument block; no HIP call is made
// unless num_splits == 0 (the heuristic reads the device's compute-unit count).
constexpr int kMaxQueryTokens = 65536;


int prepare_decode(const kvq_cache_t *cache, const void *q, const int32_t *block_tables, int32_t max_blocks_per_seq,
                   const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                   int32_t num_splits, float *out, float *lse, const void *workspace, size_t workspace_bytes_given,
                   bool need_inputs, bool need_outputs, kvq::DecodeArgs &a, int nq = 1) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  st = check_heads(cache, num_q_heads);
  if (st != KVQ_OK) return st;
  if (nq < 1 || nq > kMaxQueryTokens) return KVQ_ERR_INVALID_ARG;
  if (nq > 1 && cache->dtype == KVQ_BF16) return KVQ_ERR_UNSUPPORTED;
  if (num_seqs <= 0 || (need_inputs && max_blocks_per_seq <= 0)) return KVQ_ERR_INVALID_ARG;
  if (max_context_len < 1 || (need_inputs && (int64_t)max_context_len > (int64_t)max_blocks_per_seq * kvq::kPage))
    return KVQ_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > kMaxSplits) return KVQ_ERR_INVALID_ARG;
  if (!context_lens || !workspace || !aligned(context_lens, 4) || !aligned(workspace, 256)) return KVQ_ERR_INVALID_ARG;
  if (need_inputs && (!q || !block_tables || !aligned(q, 16) || !aligned(block_tables, 4))) return KVQ_ERR_INVALID_ARG;
  if (need_outputs && (!out || !aligned(out, 16) || (lse && !aligned(lse, 4)))) return KVQ_ERR_INVALID_ARG;
  const int D = cache->head_dim, Hkv = cache->num_kv_heads;
  const int Gq = num_q_heads / Hkv;
  const int RT = row_tiles_for(nq, Gq), CH = chunks_for(nq, Gq);
  const int NS = num_splits ? num_splits
                            : choose_splits(cache->dtype, num_seqs, Hkv, D, max_context_len, device_cus(), RT, CH);
  const int RTW = rtw_for(RT), RG = (RT + RTW - 1) / RTW;
  if ((int64_t)num_seqs * CH * Hkv * NS * RG > INT32_MAX ||
      (int64_t)num_seqs * nq * num_q_heads * (D / 64) > INT32_MAX)
    return KVQ_ERR_INVALID_ARG;
  // one sequence's query block and partials are addressed with 32-bit buffer offsets
  if (nq > 1 && ((int64_t)nq * num_q_heads * NS * D * 4 >= INT32_MAX || (int64_t)nq * num_q_heads * D * 2 >= INT32_MAX))
    return KVQ_ERR_INVALID_ARG;
  if (workspace_bytes_given < workspace_bytes(num_seqs * nq, num_q_heads, NS, D)) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  const int64_t max_pages = ((int64_t)max_context_len + kvq::kPage - 1) / kvq::kPage;
  a.q = static_cast<const uint16_t *>(q);
  a.kc = cache->k;
  a.vc = cache->v;
  a.ks = static_cast<const uint16_t *>(cache->k_scales);
  a.vs = static_cast<const uint16_t *>(cache->v_scales);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t rows = (size_t)num_seqs * nq * num_q_heads * NS;
  const size_t o_bytes = (rows * D * sizeof(float) + 255) & ~(size_t)255;
  a.o_part = static_cast<float *>(const_cast<void *>(workspace));
  a.ml = reinterpret_cast<float2 *>(static_cast<char *>(const_cast<void *>(workspace)) + o_bytes);
  a.out = out;
  a.lse = lse;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.max_blocks = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.S = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = Hkv;
  a.G = num_q_heads / Hkv;
  a.NB = cache->num_blocks;
  a.NS = NS;
  a.cpp = (int)((max_pages + NS - 1) / NS);
  a.D = D;
  a.waves = waves_for(cache->dtype, D);
  a.nq = nq;
  a.qchunk = qchunk_for(nq, Gq);
  a.chunks = CH;
  a.int_qk = 0;
  a.row_tiles = RT;
  a.rtw = RTW;
  a.row_groups = RG;
  return KVQ_OK;
}

// k_new / v_new: the step's new tokens (fused quantize-on-write), or null for attention only.
int decode_impl(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q,
                const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, float *out,
                float *lse, void *workspace, size_t workspace_bytes_given, void *stream) {
  kvq::DecodeArgs a;
  int st = prepare_decode(cache, q, block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                          num_q_heads, num_splits, out, lse, workspace, workspace_bytes_given, true, true, a);
  if (st != KVQ_OK) return st;
  if ((k_new == nullptr) != (v_new == nullptr)) return KVQ_ERR_INVALID_ARG;
  if (k_new && (!aligned(k_new, 16) || !aligned(v_new, 16))) return KVQ_ERR_INVALID_ARG;
  a.k_new = static_cast<const uint16_t *>(k_new);
  a.v_new = static_cast<const uint16_t *>(v_new);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kvq::launch_decode_split(cache->dtype, a, s) != hipSuccess) return KVQ_ERR_LAUNCH_FAILED;
  if (kvq::launch_decode_merge(a, s) != hipSuccess) return KVQ_ERR_LAUNCH_FAILED;
  return KVQ_OK;
}

int write_impl(const kvq_cache_t *cache, const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
               void *stream) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (num_tokens < 0) return KVQ_ERR_INVALID_ARG;
  if (num_tokens == 0) return KVQ_OK;
  if (!k || !v || !slot_mapping || !aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 4))
    return KVQ_ERR_INVALID_ARG;
  const int per = cache->dtype == KVQ_INT8_Q8_0   ? 2 * (cache->head_dim / kvq::kGroup)
                  : cache->dtype == KVQ_BF16 ? 2 * (cache->head_dim / 8)
                                             : 2;  // per-head: one wavefront per row
  if ((int64_t)num_tokens * cache->num_kv_heads * per > (int64_t)INT32_MAX * 256) return KVQ_ERR_INVALID_ARG;
  kvq::WriteArgs a;
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.slot_mapping = slot_mapping;
  a.kc = cache->k;
  a.vc = cache->v;
  a.ks = static_cast<uint16_t *>(cache->k_scales);
  a.vs = static_cast<uint16_t *>(cache->v_scales);
  a.T = num_tokens;
  a.Hkv = cache->num_kv_heads;
  a.D = cache->head_dim;
  a.NB = cache->num_blocks;
  hipError_t e = kvq::launch_kv_write(cache->dtype, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH_FAILED;
}

template <typename T>
bool to_host(std::vector<T> &dst, const void *src, size_t n, hipStream_t st) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, st) != hipSuccess) return false;
  return hipStreamSynchronize(st) == hipSuccess;
}

bool all_finite(const std::vector<uint16_t> &x) {
  for (uint16_t b : x)
    if (!bf16_finite(b)) return false;
  return true;
}

// Checked mode of decode (and of the fused step when k_new != null): host copies of the metadata
// and inputs, validated against the contract, then the fast path and a synchronisation.
int check_decode_impl(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q,
                      const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                      int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, float *out,
                      float *lse, void *workspace, size_t workspace_bytes_given, void *stream) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  st = check_heads(cache, num_q_heads);
  if (st != KVQ_OK) return st;
  if (num_seqs <= 0 || max_blocks_per_seq <= 0 || !q || !block_tables || !context_lens) return KVQ_ERR_INVALID_ARG;
  if (max_context_len < 1 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * kvq::kPage)
    return KVQ_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (is_capturing(s)) return KVQ_ERR_CAPTURING;
  std::vector<int32_t> lens, tables;
  if (!to_host(lens, context_lens, (size_t)num_seqs, s)) return KVQ_ERR_LAUNCH_FAILED;
  if (!to_host(tables, block_tables, (size_t)num_seqs * max_blocks_per_seq, s)) return KVQ_ERR_LAUNCH_FAILED;
  std::unordered_set<int32_t> new_blocks;
  for (int i = 0; i < num_seqs; ++i) {
    const int32_t L = lens[i];
    if (L < 0 || L > max_context_len) return KVQ_ERR_VALIDATION_FAILED;
    const int pages = (int)(((int64_t)L + kvq::kPage - 1) / kvq::kPage);
    for (int p = 0; p < pages; ++p) {
      const int32_t b = tables[(size_t)i * max_blocks_per_seq + p];
      if (b < 0 || b >= cache->num_blocks) return KVQ_ERR_VALIDATION_FAILED;
    }
    if (k_new && pages > 0 && !new_blocks.insert(tables[(size_t)i * max_blocks_per_seq + pages - 1]).second)
      return KVQ_ERR_VALIDATION_FAILED;  // two sequences write into one block
  }
  if (k_new) {  // no other sequence may read a block that receives a new token
    for (int i = 0; i < num_seqs; ++i) {
      const int pages = (int)(((int64_t)lens[i] + kvq::kPage - 1) / kvq::kPage);
      for (int p = 0; p + 1 < pages; ++p)
        if (new_blocks.count(tables[(size_t)i * max_blocks_per_seq + p])) return KVQ_ERR_VALIDATION_FAILED;
    }
  }
  std::vector<uint16_t> hq;
  if (!to_host(hq, q, (size_t)num_seqs * num_q_heads * cache->head_dim, s)) return KVQ_ERR_LAUNCH_FAILED;
  if (!all_finite(hq)) return KVQ_ERR_VALIDATION_FAILED;
  if (k_new) {
    if (!v_new) return KVQ_ERR_INVALID_ARG;
    std::vector<uint16_t> hk, hv;
    const size_t n = (size_t)num_seqs * cache->num_kv_heads * cache->head_dim;
    if (!to_host(hk, k_new, n, s) || !to_host(hv, v_new, n, s)) return KVQ_ERR_LAUNCH_FAILED;
    if (!all_finite(hk) || !all_finite(hv)) return KVQ_ERR_VALIDATION_FAILED;
  }
  st = decode_impl(cache, k_new, v_new, q, block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                   num_q_heads, num_splits, out, lse, workspace, workspace_bytes_given, stream);
  if (st != KVQ_OK) return st;
  return hipStreamSynchronize(s) == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH_FAILED;
}

}  // namespace

extern "C" {

int kvq_write(const kvq_cache_t *cache, const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
              void *stream) {
  return write_impl(cache, k, v, slot_mapping, num_tokens, stream);
}

size_t kvq_decode_workspace_bytes(const kvq_cache_t *cache, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_splits) {
  if (check_cache(cache) != KVQ_OK || check_heads(cache, num_q_heads) != KVQ_OK) return 0;
  if (num_seqs <= 0 || num_splits <= 0 || num_splits > kMaxSplits) return 0;
  return workspace_bytes(num_seqs, num_q_heads, num_splits, cache->head_dim);
}

int32_t kvq_choose_num_splits(const kvq_cache_t *cache, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_context_len) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  st = check_heads(cache, num_q_heads);
  if (st != KVQ_OK) return st;
  if (num_seqs <= 0 || max_context_len < 1) return KVQ_ERR_INVALID_ARG;
  return choose_splits(cache->dtype, num_seqs, cache->num_kv_heads, cache->head_dim, max_context_len, device_cus());
}

int32_t kvq_choose_num_splits_lengths(const kvq_cache_t *cache, int32_t num_seqs, int32_t num_q_heads,
                                      const int32_t *host_context_lens) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  st = check_heads(cache, num_q_heads);
  if (st != KVQ_OK) return st;
  if (num_seqs <= 0 || !host_context_lens) return KVQ_ERR_INVALID_ARG;
  for (int s = 0; s < num_seqs; ++s)
    if (host_context_lens[s] < 0) return KVQ_ERR_INVALID_ARG;
  return choose_splits_lengths(cache->dtype, num_seqs, cache->num_kv_heads, cache->head_dim, host_context_lens,
                               device_cus());
}

int kvq_decode_attention(const kvq_cache_t *cache, const void *q, const int32_t *block_tables,
                         int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, float *out, float *lse,
                         void *workspace, size_t workspace_bytes_given, void *stream) {
  return decode_impl(cache, nullptr, nullptr, q, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                     num_seqs, num_q_heads, num_splits, out, lse, workspace, workspace_bytes_given, stream);
}

int kvq_decode_attention_int8qk(const kvq_cache_t *cache, const void *q, const int32_t *block_tables,
                                int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                                int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, float *out, float *lse,
                                void *workspace, size_t workspace_bytes_given, void *stream) {
  kvq::DecodeArgs a;
  int st = prepare_decode(cache, q, block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                          num_q_heads, num_splits, out, lse, workspace, workspace_bytes_given, true, true, a);
  if (st != KVQ_OK) return st;
  if (cache->dtype != KVQ_INT8_Q8_0) return KVQ_ERR_UNSUPPORTED;
  a.int_qk = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kvq::launch_decode_split(cache->dtype, a, s) != hipSuccess) return KVQ_ERR_LAUNCH_FAILED;
  if (kvq::launch_decode_merge(a, s) != hipSuccess) return KVQ_ERR_LAUNCH_FAILED;
  return KVQ_OK;
}

int kvq_decode_attention_mq(const kvq_cache_t *cache, const void *q, int32_t num_query_tokens,
                            const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits,
                            float *out, float *lse, void *workspace, size_t workspace_bytes_given, void *stream) {
  kvq::DecodeArgs a;
  int st = prepare_decode(cache, q, block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                          num_q_heads, num_splits, out, lse, workspace, workspace_bytes_given, true, true, a,
                          num_query_tokens);
  if (st != KVQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kvq::launch_decode_split(cache->dtype, a, s) != hipSuccess) return KVQ_ERR_LAUNCH_FAILED;
  if (kvq::launch_decode_merge(a, s) != hipSuccess) return KVQ_ERR_LAUNCH_FAILED;
  return KVQ_OK;
}

int32_t kvq_choose_num_splits_mq(const kvq_cache_t *cache, int32_t num_seqs, int32_t num_query_tokens,
                                 int32_t num_q_heads, int32_t max_context_len) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  st = check_heads(cache, num_q_heads);
  if (st != KVQ_OK) return st;
  if (num_seqs <= 0 || max_context_len < 1 || num_query_tokens < 1 || num_query_tokens > kMaxQueryTokens)
    return KVQ_ERR_INVALID_ARG;
  const int G = num_q_heads / cache->num_kv_heads;
  return choose_splits(cache->dtype, num_seqs, cache->num_kv_heads, cache->head_dim, max_context_len, device_cus(),
                       row_tiles_for(num_query_tokens, G), chunks_for(num_query_tokens, G));
}

int kvq_decode_step(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q,
                    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                    int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, float *out,
                    float *lse, void *workspace, size_t workspace_bytes_given, void *stream) {
  if (!k_new || !v_new) return KVQ_ERR_INVALID_ARG;
  return decode_impl(cache, k_new, v_new, q, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                     num_seqs, num_q_heads, num_splits, out, lse, workspace, workspace_bytes_given, stream);
}

int kvq_decode_step_noalloc(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q,
                            const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits,
                            float *out, float *lse, void *stream) {
  if (!k_new || !v_new) return KVQ_ERR_INVALID_ARG;
  // size check before the scratch is looked up: a call that needs more than the fixed buffer is
  // refused with nothing enqueued
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  st = check_heads(cache, num_q_heads);
  if (st != KVQ_OK) return st;
  if (num_seqs <= 0 || max_context_len < 1 || num_splits < 0 || num_splits > kMaxSplits) return KVQ_ERR_INVALID_ARG;
  const int ns = num_splits ? num_splits
                            : choose_splits(cache->dtype, num_seqs, cache->num_kv_heads, cache->head_dim,
                                            max_context_len, device_cus());
  if (workspace_bytes(num_seqs, num_q_heads, ns, cache->head_dim) > kvq::kScratchBytes)
    return KVQ_ERR_WORKSPACE_TOO_SMALL;
  void *scratch = nullptr;
  if (kvq::scratch_address(&scratch) != hipSuccess) return KVQ_ERR_LAUNCH_FAILED;
  return decode_impl(cache, k_new, v_new, q, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                     num_seqs, num_q_heads, ns, out, lse, scratch, kvq::kScratchBytes, stream);
}

size_t kvq_decode_step_noalloc_max_bytes(void) { return kvq::kScratchBytes; }

int kvq_check_decode_step(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q,
                          const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                          int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits,
                          float *out, float *lse, void *workspace, size_t workspace_bytes_given, void *stream) {
  if (!k_new || !v_new) return KVQ_ERR_INVALID_ARG;
  return check_decode_impl(cache, k_new, v_new, q, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                           num_seqs, num_q_heads, num_splits, out, lse, workspace, workspace_bytes_given, stream);
}

int kvq_decode_partials(const kvq_cache_t *cache, const void *q, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, void *workspace,
                        size_t workspace_bytes_given, void *stream) {
  kvq::DecodeArgs a;
  int st = prepare_decode(cache, q, block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                          num_q_heads, num_splits, nullptr, nullptr, workspace, workspace_bytes_given, true, false, a);
  if (st != KVQ_OK) return st;
  return kvq::launch_decode_split(cache->dtype, a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? KVQ_OK
             : KVQ_ERR_LAUNCH_FAILED;
}

int kvq_decode_merge(const kvq_cache_t *cache, const int32_t *context_lens, int32_t max_context_len,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, const void *workspace,
                     size_t workspace_bytes_given, float *out, float *lse, void *stream) {
  kvq::DecodeArgs a;
  int st = prepare_decode(cache, nullptr, nullptr, 0, context_lens, max_context_len, num_seqs, num_q_heads,
                          num_splits, out, lse, workspace, workspace_bytes_given, false, true, a);
  if (st != KVQ_OK) return st;
  return kvq::launch_decode_merge(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KVQ_OK
                                                                                      : KVQ_ERR_LAUNCH_FAILED;
}

int kvq_check_write(const kvq_cache_t *cache, const void *k, const void *v, const int32_t *slot_mapping,
                    int32_t num_tokens, void *stream) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (num_tokens < 0) return KVQ_ERR_INVALID_ARG;
  if (num_tokens == 0) return KVQ_OK;
  if (!k || !v || !slot_mapping) return KVQ_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (is_capturing(s)) return KVQ_ERR_CAPTURING;
  std::vector<int32_t> slots;
  if (!to_host(slots, slot_mapping, (size_t)num_tokens, s)) return KVQ_ERR_LAUNCH_FAILED;
  std::unordered_set<int32_t> seen;
  const int64_t nslots = (int64_t)cache->num_blocks * kvq::kPage;
  for (int32_t x : slots) {
    if (x < 0) continue;
    if (x >= nslots) return KVQ_ERR_VALIDATION_FAILED;
    if (!seen.insert(x).second) return KVQ_ERR_VALIDATION_FAILED;
  }
  const size_t n = (size_t)num_tokens * cache->num_kv_heads * cache->head_dim;
  std::vector<uint16_t> hk, hv;
  if (!to_host(hk, k, n, s) || !to_host(hv, v, n, s)) return KVQ_ERR_LAUNCH_FAILED;
  for (size_t i = 0; i < n; ++i)
    if (!bf16_finite(hk[i]) || !bf16_finite(hv[i])) return KVQ_ERR_VALIDATION_FAILED;
  st = write_impl(cache, k, v, slot_mapping, num_tokens, stream);
  if (st != KVQ_OK) return st;
  return hipStreamSynchronize(s) == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH_FAILED;
}

int kvq_check_decode(const kvq_cache_t *cache, const void *q, const int32_t *block_tables,
                     int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, float *out, float *lse,
                     void *workspace, size_t workspace_bytes_given, void *stream) {
  return check_decode_impl(cache, nullptr, nullptr, q, block_tables, max_blocks_per_seq, context_lens,
                           max_context_len, num_seqs, num_q_heads, num_splits, out, lse, workspace,
                           workspace_bytes_given, stream);
}

int32_t kvq_page_offset(int32_t dtype, int32_t head_dim, int32_t which, int32_t token, int32_t channel) {
  if ((head_dim != 128 && head_dim != 256) || token < 0 || token >= kvq::kPage || channel < 0 ||
      channel >= head_dim || (which != 0 && which != 1))
    return -1;
  if (dtype == KVQ_INT8_Q8_0 || dtype == KVQ_INT8_PER_HEAD)
    return (int32_t)(which ? kvq::i8_v_offset(token, channel) : kvq::i8_k_offset(token, channel));
  if (dtype == KVQ_BF16)
    return (int32_t)(which ? kvq::bf16_v_offset(token, channel) : kvq::bf16_k_offset(token, channel));
  return -1;
}

const char *kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARG: return "KVQ_ERR_INVALID_ARG";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_WORKSPACE_TOO_SMALL: return "KVQ_ERR_WORKSPACE_TOO_SMALL";
    case KVQ_ERR_LAUNCH_FAILED: return "KVQ_ERR_LAUNCH_FAILED";
    case KVQ_ERR_VALIDATION_FAILED: return "KVQ_ERR_VALIDATION_FAILED";
    case KVQ_ERR_CAPTURING: return "KVQ_ERR_CAPTURING";
    default: return "KVQ_ERR_UNKNOWN";
  }
}

}  // extern "C"
