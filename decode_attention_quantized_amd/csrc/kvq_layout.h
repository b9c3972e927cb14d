// In-page layouts of the paged KV cache, shared by the kernels and the host API.
//
// A page holds 16 tokens of one KV head.  Its bytes are ordered so that every lane of a
// 64-wide wavefront receives exactly its MFMA operand fragment with one 16-byte load per
// instruction, and every load instruction of a wavefront reads 1 KiB of contiguous memory.
//
// INT8 K page (QK^T: A operand = K codes, 16 tokens x 32 channels of one scale group per
//   v_mfma_f32_16x16x32_f16; lane l = 16*q + t holds token t, channels 32g + 8q + 0..7):
//   load i (0 .. D/64-1) of lane l brings channels of groups 2i and 2i+1.
// INT8 V page (P.V: B operand = V codes, K-slots are tokens; lane l = 16*qt + n holds the
//   4 tokens 4qt..4qt+3 of channel 16*jt + n for tile jt): load k brings tiles 4k..4k+3.
// BF16 pages use the same scheme with 2-byte elements (16 bytes = 8 bf16 values).
#pragma once

#include <stdint.h>

namespace kvq {

constexpr int kPage = 16;   // tokens per page
constexpr int kGroup = 32;  // values per scale

__host__ __device__ inline uint32_t i8_k_offset(int t, int c) {
  return ((((uint32_t)(c >> 6) << 6) | ((uint32_t)((c >> 3) & 3) << 4) | (uint32_t)t) << 4) |
         ((uint32_t)((c >> 5) & 1) << 3) | (uint32_t)(c & 7);
}

__host__ __device__ inline uint32_t i8_v_offset(int t, int c) {
  return ((((uint32_t)(c >> 6) << 6) | ((uint32_t)(t >> 2) << 4) | (uint32_t)(c & 15)) << 4) |
         ((uint32_t)((c >> 4) & 3) << 2) | (uint32_t)(t & 3);
}

__host__ __device__ inline uint32_t bf16_k_offset(int t, int c) {
  return ((((uint32_t)(c >> 5) << 6) | ((uint32_t)((c >> 3) & 3) << 4) | (uint32_t)t) << 3) | (uint32_t)(c & 7);
}

__host__ __device__ inline uint32_t bf16_v_offset(int t, int c) {
  return ((((uint32_t)(c >> 5) << 6) | ((uint32_t)(t >> 2) << 4) | (uint32_t)(c & 15)) << 3) |
         ((uint32_t)((c >> 4) & 1) << 2) | (uint32_t)(t & 3);
}

}  // namespace kvq
