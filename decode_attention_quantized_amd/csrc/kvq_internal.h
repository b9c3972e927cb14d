// Internal interface between the C ABI (kvq_api.cpp) and the kernels (kvq_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct WriteArgs {
  const uint16_t *k, *v;          // bf16 [T][Hkv][D]
  const int32_t *slot_mapping;    // [T]
  void *kc, *vc;                  // code / value planes
  uint16_t *ks, *vs;              // scale planes: fp16 (q8_0) or fp32 (per-head, as uint16_t pairs)
  int T, Hkv, D, NB;
};

struct DecodeArgs {
  const uint16_t *q;              // bf16 [S][Hq][D]
  const void *kc, *vc;            // code / value planes
  const uint16_t *ks, *vs;        // scale planes: fp16 (q8_0) or fp32 (per-head); null for BF16
  const int32_t *block_tables;    // [S][max_blocks]
  const int32_t *context_lens;    // [S]
  float *o_part;                  // workspace: fp32 [S][Hq][NS][D]
  float2 *ml;                     // workspace: (max in log2 units, sum) [S][Hq][NS]
  float *out;                     // fp32 [S][Hq][D]
  float *lse;                     // fp32 [S][Hq] or null
  const uint16_t *k_new, *v_new;  // bf16 [S][Hkv][D]: token context_len-1 of each sequence, quantized
                                  // into its page by the split kernel before the page is read (or null)
  int max_blocks, max_context_len, S, Hq, Hkv, G, NB, NS, cpp, D;
  int waves;                      // wavefronts per split workgroup (1, 2, 4 or 8)
  int nq;                         // query tokens per sequence (q [S][nq][Hq][D], causal among them)
  int qchunk;                     // query tokens per workgroup (the chunk; nq is cut into chunks)
  int chunks;                     // ceil(nq / qchunk)
  int int_qk;                     // 1: integer Q.K (Q quantized per 32 values like the cache; q8_0 only)
  int row_tiles;                  // ceil(qchunk * G / 16): 16-row MFMA tiles of (query token, head) pairs
  int rtw;                        // row tiles per workgroup (1, 2 or 4; its waves split into rtw groups)
  int row_groups;                 // ceil(row_tiles / rtw): workgroups per (split, KV head, sequence)
};

// Bytes of the fixed device scratch used by kvq_decode_step_noalloc (the split partials).
constexpr size_t kScratchBytes = (size_t)8 << 20;

// Device address of the current device's fixed scratch (looked up once per device).
hipError_t scratch_address(void **ptr);

// Each returns hipSuccess or the launch error.  dtype: 0 INT8 q8_0, 1 BF16, 2 INT8 per-head.
hipError_t launch_kv_write(int dtype, const WriteArgs &a, hipStream_t stream);
hipError_t launch_decode_split(int dtype, const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t stream);

}  // namespace kvq
