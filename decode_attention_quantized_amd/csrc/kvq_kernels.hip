// HIP kernels for gfx950 (MI355X): quantize-on-write, split-KV GQA decode attention over the
// paged INT8 (or BF16) cache, and the log-sum-exp merge of the split partials.
//
// Quantize-on-write follows the q8_0-style rule of the half-the-memory page (section "Is 8
// bits enough?": one scale per 32 values) and the gllm page (section "Quantization Design":
// amax/127, round to nearest, clamp to +-127).  Split-KV follows the long-context page
// (section "Give more GPU workers a piece of the attention calculation"): each workgroup
// handles a contiguous range of pages of one (sequence, KV head), keeps a running maximum
// and normalisation sum (online softmax) and writes an unnormalised partial; the merge
// combines partials with those terms.  The cache is read directly, dequantized in registers
// (half-the-memory page, section "Read the compressed cache without copying it first").
//
// Numerics.  Q.K: K codes (exact in f16) times Q (bf16 rescaled by a power of two per head
// so that it is exact in f16) on v_mfma_f32_16x16x32_f16, one MFMA per 32-channel scale
// group, fp32 accumulation, then the fp16 group scale applied in fp32.  P.V: P' = p * s_v
// per (token, group) split into f16 hi + lo parts (about 22 significant bits), times exact
// f16 V codes on the same MFMA.  Softmax in base 2 with log2(e)/sqrt(D) folded into one
// multiply per score.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "kvq_internal.h"
#include "kvq_layout.h"

namespace kvq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef int v4i_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Four int8 codes (one dword) -> four exact f16 values, as two f16x2 words.
// (x ^ 0x80) is x + 128 as an unsigned byte u; v_perm places u under the exponent byte 0x64,
// giving the f16 value 1024 + u; subtracting 1152 (one packed f16 add) gives x exactly.
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, uint32_t &lo, uint32_t &hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // bytes 0, 1
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // bytes 2, 3
  const h2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, a) + bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, b) + bias);
}

// Eight int8 codes (two dwords) -> the f16x8 MFMA operand, element e = byte e.
__device__ __forceinline__ h8_t i8x8_to_h8(uint32_t w0, uint32_t w1) {
  uint32_t r0, r1, r2, r3;
  i8x4_to_f16(w0, r0, r1);
  i8x4_to_f16(w1, r2, r3);
  return __builtin_bit_cast(h8_t, u4_t{r0, r1, r2, r3});
}

__device__ __forceinline__ f4_t mfma_f16(h8_t a, h8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The K = 16 form: a lane's four K slots are its own four rows of B (four tokens of a page).
__device__ __forceinline__ f4_t mfma16_f16(h4_t a, h4_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4_t mfma_bf16(b8_t a, b8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fma(s, b, c) with s the fp16 number in the low / high half of h2 (exact widening; the
// compiler emits one v_fma_mix_f32).
__device__ __forceinline__ float fma_h16lo(uint32_t h2, float b, float c) {
  return fmaf(f16_bits_to_f32(h2 & 0xFFFFu), b, c);
}
__device__ __forceinline__ float fma_h16hi(uint32_t h2, float b, float c) { return fmaf(f16_bits_to_f32(h2 >> 16), b, c); }

// Makes the values available at this point of the program (an empty asm that passes them
// through), so that the compiler cannot defer the work that produces them past later code.
// Not volatile: it has no side effects and leaves the block-table loads scalar.
__device__ __forceinline__ void pin4(f4_t &v) {
  float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
  asm("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
  v = f4_t{a0, a1, a2, a3};
}

// ------------------------------------------------------------------ quantize-on-write

// The fp16 scale of a group with maximum magnitude amax: fp16(min(amax / 127, 65504)), an fp32
// division and a round to nearest even.
__device__ __forceinline__ _Float16 q8_scale(float amax) { return (_Float16)fminf(amax / 127.0f, 65504.0f); }

// The codes of N values against the stored scale s (as fp32): rint(x / s) (nearest even) clamped
// to +-127; 0 when s is 0 or x / s is NaN.  Packed four to a word, byte e % 4 of word e / 4.
// x * (1 / s), with 1 / s correctly rounded, lies within 1.5 * 2^-23 |x / s| of the correctly
// rounded quotient x / s, so for |x / s| < 256 (above that both clamp) the two round to the same
// integer unless x * (1 / s) is within 2^-12 of a half-integer.  Only such values, and values
// where the product is not finite (1 / s overflows for an fp32 scale below 2^-128), take the
// quotient itself, in a block that a lane enters only when it holds one.
template <int N>
__device__ __forceinline__ void q8_codes(const float *x, float s, uint32_t *packed) {
  const float rs = 1.0f / s;
  float q[N];
  bool near = false;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    q[e] = x[e] * rs;
    near |= !(fabsf(__builtin_amdgcn_fractf(q[e]) - 0.5f) >= 0x1p-12f);  // NaN: not finite
  }
  if (__builtin_expect(near, 0)) {
#pragma unroll
    for (int e = 0; e < N; ++e)
      if (!(fabsf(__builtin_amdgcn_fractf(q[e]) - 0.5f) >= 0x1p-12f)) q[e] = x[e] / s;
  }
#pragma unroll
  for (int w = 0; w < N / 4; ++w) packed[w] = 0u;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    float r = __builtin_rintf(q[e]);
    r = (r != r) ? 0.0f : fminf(fmaxf(r, -127.0f), 127.0f);
    r = (s != 0.0f) ? r : 0.0f;
    packed[e >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (e & 3));
  }
}

// The same codes from the quotient itself, with no branch: for the quantization inside the
// decode kernels, whose prologue the compiler schedules as one straight block.
template <int N>
__device__ __forceinline__ void q8_codes_div(const float *x, float s, uint32_t *packed) {
#pragma unroll
  for (int w = 0; w < N / 4; ++w) packed[w] = 0u;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    float r = __builtin_rintf(x[e] / s);
    r = (r != r) ? 0.0f : fminf(fmaxf(r, -127.0f), 127.0f);
    r = (s != 0.0f) ? r : 0.0f;
    packed[e >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (e & 3));
  }
}

// The writers take the inputs of their first memory requests (the bf16 rows, the slot mapping and
// the sizes that place a workgroup) as leading scalar arguments, preloaded into scalar registers at
// launch; the plane pointers, needed only for the stores, come from the argument block.
#define KVQ_WRITE_PARAMS                                                                              \
  const uint16_t *__restrict__ k_rows, const uint16_t *__restrict__ v_rows, const int32_t *__restrict__ slots, \
      int num_tokens, int num_kv_heads
__device__ __forceinline__ WriteArgs write_placed(const WriteArgs &args, const uint16_t *k_rows,
                                                  const uint16_t *v_rows, const int32_t *slots, int num_tokens,
                                                  int num_kv_heads) {
  WriteArgs a = args;
  a.k = k_rows;
  a.v = v_rows;
  a.slot_mapping = slots;
  a.T = num_tokens;
  a.Hkv = num_kv_heads;
  return a;
}
#define KVQ_WRITE_PLACED(args) write_placed(args, k_rows, v_rows, slots, num_tokens, num_kv_heads)

// Few tokens (fewer than a page: the step of a decode batch): one thread per (token, KV head,
// K or V, 32-channel group), each storing its group's codes straight into the page.
template <int D>
__global__ __launch_bounds__(256) void kv_write_i8_rows_kernel(KVQ_WRITE_PARAMS, WriteArgs args) {
  const WriteArgs a = KVQ_WRITE_PLACED(args);
  constexpr int NG = D / kGroup;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.T * a.Hkv * 2 * NG;
  if (gid >= total) return;
  const int g = (int)(gid % NG);
  int64_t r = gid / NG;
  const int which = (int)(r & 1);
  r >>= 1;
  const int h = (int)(r % a.Hkv);
  const int t = (int)(r / a.Hkv);
  const int32_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.NB * kPage) return;
  const int blk = slot >> 4, off = slot & 15;

  const u4_t *src = reinterpret_cast<const u4_t *>((which ? a.v : a.k) + ((int64_t)t * a.Hkv + h) * D + g * kGroup);
  float x[kGroup];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u4_t w = src[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * i + 2 * e] = bf16_lo(w[e]);
      x[8 * i + 2 * e + 1] = bf16_hi(w[e]);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const _Float16 s16 = q8_scale(amax);
  const float s = (float)s16;
  uint32_t packed[kGroup / 4];
  q8_codes<kGroup>(x, s, packed);
  const int64_t page = (int64_t)blk * a.Hkv + h;
  const uint16_t sbits = __builtin_bit_cast(uint16_t, s16);
  if (which == 0) {
    int8_t *dst = static_cast<int8_t *>(a.kc) + page * (kPage * D);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      u2_t w = {packed[2 * qq], packed[2 * qq + 1]};
      *reinterpret_cast<u2_t *>(dst + i8_k_offset(off, kGroup * g + 8 * qq)) = w;
    }
    a.ks[(page * NG + g) * kPage + off] = sbits;
  } else {
    int8_t *dst = static_cast<int8_t *>(a.vc) + page * (kPage * D);
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
      dst[i8_v_offset(off, kGroup * g + i)] = (int8_t)((packed[i >> 2] >> (8 * (i & 3))) & 0xFFu);
    a.vs[(page * NG + g) * kPage + off] = sbits;
  }
}

// BF16 cache, few tokens: one thread per (token, KV head, K or V, 8-channel chunk); a scatter copy.
template <int D>
__global__ __launch_bounds__(256) void kv_write_bf16_rows_kernel(KVQ_WRITE_PARAMS, WriteArgs args) {
  const WriteArgs a = KVQ_WRITE_PLACED(args);
  constexpr int NC = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.T * a.Hkv * 2 * NC;
  if (gid >= total) return;
  const int cchunk = (int)(gid % NC);
  int64_t r = gid / NC;
  const int which = (int)(r & 1);
  r >>= 1;
  const int h = (int)(r % a.Hkv);
  const int t = (int)(r / a.Hkv);
  const int32_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.NB * kPage) return;
  const int blk = slot >> 4, off = slot & 15;
  const u4_t w = *reinterpret_cast<const u4_t *>((which ? a.v : a.k) + ((int64_t)t * a.Hkv + h) * D + 8 * cchunk);
  const int64_t page = (int64_t)blk * a.Hkv + h;
  const int c0 = 8 * cchunk;
  if (which == 0) {
    uint16_t *dst = static_cast<uint16_t *>(a.kc) + page * (kPage * D);
    *reinterpret_cast<u4_t *>(dst + bf16_k_offset(off, c0)) = w;
  } else {
    uint16_t *dst = static_cast<uint16_t *>(a.vc) + page * (kPage * D);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      dst[bf16_v_offset(off, c0 + e)] = (uint16_t)((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
  }
}

// Token windows.  Workgroup (b, h) owns the tokens 16b .. 16b + 15 of the batch for KV head h.
// A full page is 16 tokens t0 .. t0 + 15, consecutive in the batch, whose slots are 16p, 16p + 1,
// ..., 16p + 15 in that order (a prefill writes its pages so).  The workgroup whose window holds
// t0 writes such a page whole, with 16-byte stores of whole page rows; every other valid token
// of its window is written on its own.  At most one full page starts in a window, and no token
// lies in two: the slot of any later token of a page is not a multiple of 16.
struct WriteWindow {
  int page_t0;      // first token of the full page that starts in this window, or -1
  int page_blk;     // that page's block
  uint32_t single;  // bit t: token 16b + t has a valid slot and lies in no full page
  int32_t slot;     // lane 16 + t: the slot of token 16b + t (broadcast below)
};

// Every wave of the workgroup takes the same decision from the same 48 slots: lane l looks at
// token 16b - 16 + l and its successor.
__device__ __forceinline__ WriteWindow scan_window(const WriteArgs &a, int b, int lane) {
  const int64_t t = (int64_t)b * kPage - kPage + lane;
  const int32_t limit = a.NB * kPage;
  const int32_t s0 = (t >= 0 && t < a.T) ? a.slot_mapping[t] : -1;
  const int32_t s1 = (t + 1 >= 0 && t + 1 < a.T) ? a.slot_mapping[t + 1] : -1;
  const bool v0 = s0 >= 0 && s0 < limit;
  const uint64_t valid = __ballot(v0);
  const uint64_t aligned = __ballot(v0 && (s0 & (kPage - 1)) == 0);
  const uint64_t next = __ballot(v0 && s1 == s0 + 1);
  // bit l of run: tokens l .. l + 15 have consecutive slots (15 successor bits in a row)
  uint64_t run = next & (next >> 1);
  run &= run >> 2;
  run &= run >> 4;
  run &= run >> 7;
  const uint64_t full = aligned & run & 0xFFFFFFFFull;  // page starts at window positions 0 .. 31
  uint64_t cover = full;                                 // tokens that some full page holds
  cover |= cover << 1;
  cover |= cover << 2;
  cover |= cover << 4;
  cover |= cover << 8;
  WriteWindow w;
  const uint32_t own = (uint32_t)(full >> kPage) & 0xFFFFu;
  w.page_t0 = -1;
  w.page_blk = 0;
  if (own) {
    const int l = kPage + __builtin_ctz(own);
    w.page_t0 = b * kPage + (l - kPage);
    w.page_blk = __builtin_amdgcn_readlane(s0, l) >> 4;
  }
  w.single = (uint32_t)((valid & ~cover) >> kPage) & 0xFFFFu;
  w.slot = s0;
  return w;
}

// Lane (q, t) of wave i covers channels 64i + 8q .. 64i + 8q + 7 (scale group 2i) and
// 64i + 32 + 8q .. + 7 (group 2i + 1) of token t: two 16-byte loads of the bf16 row.
__device__ __forceinline__ void load_row_halves(const uint16_t *row, int i, int q, u4_t &xa, u4_t &xb) {
  const u4_t *p = reinterpret_cast<const u4_t *>(row + 64 * i + 8 * q);
  xa = p[0];
  xb = p[4];
}

// q8_0 codes of the lane's two 8-channel pieces; the group maxima are taken over the four lanes
// q = 0 .. 3 that share the token.  The result is the 16-byte K-page unit (group 2i's eight codes,
// then group 2i + 1's).
__device__ __forceinline__ u4_t quant_halves(u4_t xa, u4_t xb, _Float16 &sa, _Float16 &sb) {
  float a[8], c[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[2 * e] = bf16_lo(xa[e]);
    a[2 * e + 1] = bf16_hi(xa[e]);
    c[2 * e] = bf16_lo(xb[e]);
    c[2 * e + 1] = bf16_hi(xb[e]);
  }
  float ma = 0.0f, mc = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ma = fmaxf(ma, fabsf(a[e]));
    mc = fmaxf(mc, fabsf(c[e]));
  }
  ma = fmaxf(ma, __shfl_xor(ma, 16));
  mc = fmaxf(mc, __shfl_xor(mc, 16));
  ma = fmaxf(ma, __shfl_xor(ma, 32));
  mc = fmaxf(mc, __shfl_xor(mc, 32));
  sa = q8_scale(ma);
  sb = q8_scale(mc);
  uint32_t pa[2], pc[2];
  q8_codes<8>(a, (float)sa, pa);
  q8_codes<8>(c, (float)sb, pc);
  return u4_t{pa[0], pa[1], pc[0], pc[1]};
}

// The byte of code e of the unit (e < 8: channel 64i + 8q + e; else 64i + 32 + 8q + e - 8).
__device__ __forceinline__ uint32_t unit_byte(u4_t u, int e) { return (u[e >> 2] >> (8 * (e & 3))) & 0xFFu; }

// Per-head format: the codes of the lane's 16 channels against the row scale amax / 127, the
// row maximum taken over the workgroup's waves (s_max: one slot per wave and token, for K and V).
template <int NWV>
__device__ __forceinline__ void quant_rows_head(u4_t ka, u4_t kb, u4_t va, u4_t vb, float *s_max, int i, int q,
                                                int t, u4_t &ku, u4_t &vu, float &ks, float &vs) {
  float x[2][16];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[0][2 * e] = bf16_lo(ka[e]);
    x[0][2 * e + 1] = bf16_hi(ka[e]);
    x[0][8 + 2 * e] = bf16_lo(kb[e]);
    x[0][8 + 2 * e + 1] = bf16_hi(kb[e]);
    x[1][2 * e] = bf16_lo(va[e]);
    x[1][2 * e + 1] = bf16_hi(va[e]);
    x[1][8 + 2 * e] = bf16_lo(vb[e]);
    x[1][8 + 2 * e + 1] = bf16_hi(vb[e]);
  }
  float m[2] = {0.0f, 0.0f};
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) m[kv] = fmaxf(m[kv], fabsf(x[kv][e]));
    m[kv] = fmaxf(m[kv], __shfl_xor(m[kv], 16));
    m[kv] = fmaxf(m[kv], __shfl_xor(m[kv], 32));
  }
  if (q == 0) {
    s_max[i * kPage + t] = m[0];
    s_max[(NWV + i) * kPage + t] = m[1];
  }
  __syncthreads();
  float r[2];
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    r[kv] = s_max[kv * NWV * kPage + t];
#pragma unroll
    for (int w = 1; w < NWV; ++w) r[kv] = fmaxf(r[kv], s_max[(kv * NWV + w) * kPage + t]);
  }
  ks = r[0] / 127.0f;
  vs = r[1] / 127.0f;
  uint32_t pk[4], pv[4];
  q8_codes<16>(x[0], ks, pk);
  q8_codes<16>(x[1], vs, pv);
  ku = u4_t{pk[0], pk[1], pk[2], pk[3]};
  vu = u4_t{pv[0], pv[1], pv[2], pv[3]};
}

// INT8 caches: blockDim D (D / 64 waves), grid (windows, KV heads).  FMT 0: q8_0 (an fp16 scale per
// 32 values); FMT 1: one fp32 scale per (token, KV head).  V pages are staged in LDS: a token's
// codes spread over the V page at a 4-byte stride, so a whole page is stored at once.
template <int D, int FMT>
__global__ __launch_bounds__(D) void kv_write_i8_kernel(KVQ_WRITE_PARAMS, WriteArgs args) {
  const WriteArgs a = KVQ_WRITE_PLACED(args);
  constexpr int NG = D / kGroup;
  constexpr int NWV = D / 64;
  __shared__ __attribute__((aligned(16))) uint8_t s_v[kPage * D];
  __shared__ float s_max[2][2 * NWV * kPage];  // FMT 1: row maxima, one region per path
  const int b = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, i = threadIdx.x >> 6, q = lane >> 4, t = lane & 15;
  const WriteWindow w = scan_window(a, b, lane);
  const int64_t row_stride = (int64_t)a.Hkv * D;
  int8_t *kc = static_cast<int8_t *>(a.kc), *vc = static_cast<int8_t *>(a.vc);

  // The quantized unit pair of token `tok` and the scale stores of its lane.
  auto quant = [&](int64_t tok, int path, u4_t &ku, u4_t &vu, uint32_t &ksb, uint32_t &vsb) {
    u4_t ka, kb, va, vb;
    load_row_halves(a.k + tok * row_stride + h * D, i, q, ka, kb);
    load_row_halves(a.v + tok * row_stride + h * D, i, q, va, vb);
    if constexpr (FMT == 0) {
      _Float16 ksa, ksb2, vsa, vsb2;
      ku = quant_halves(ka, kb, ksa, ksb2);
      vu = quant_halves(va, vb, vsa, vsb2);
      ksb = __builtin_bit_cast(uint16_t, q ? ksb2 : ksa);  // lanes q = 0, 1 store groups 2i, 2i + 1
      vsb = __builtin_bit_cast(uint16_t, q ? vsb2 : vsa);
    } else {
      float ks, vs;
      quant_rows_head<NWV>(ka, kb, va, vb, s_max[path], i, q, t, ku, vu, ks, vs);
      ksb = __float_as_uint(ks);
      vsb = __float_as_uint(vs);
    }
  };
  auto store_scales = [&](int64_t page, int tt, uint32_t ksb, uint32_t vsb) {
    if constexpr (FMT == 0) {
      if (q < 2) {
        const int64_t so = (page * NG + 2 * i + q) * kPage + tt;
        a.ks[so] = (uint16_t)ksb;
        a.vs[so] = (uint16_t)vsb;
      }
    } else {
      if (i == 0 && q < 2) reinterpret_cast<float *>(q ? a.vs : a.ks)[page * kPage + tt] = __uint_as_float(q ? vsb : ksb);
    }
  };

  if (w.page_t0 >= 0) {
    const int64_t page = (int64_t)w.page_blk * a.Hkv + h;
    u4_t ku, vu;
    uint32_t ksb, vsb;
    quant(w.page_t0 + t, 0, ku, vu, ksb, vsb);
    // K unit (i, q, t) is the page's 16-byte row 64i + 16q + t = this thread's index
    *reinterpret_cast<u4_t *>(kc + page * (kPage * D) + threadIdx.x * 16) = ku;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 64 * i + 8 * q + (e & 7) + (e >> 3) * 32;
      s_v[i8_v_offset(t, c)] = (uint8_t)unit_byte(vu, e);
    }
    store_scales(page, t, ksb, vsb);
    __syncthreads();
    *reinterpret_cast<u4_t *>(vc + page * (kPage * D) + threadIdx.x * 16) =
        *reinterpret_cast<const u4_t *>(s_v + threadIdx.x * 16);
  }

  if (w.single) {
    const int64_t tok = (int64_t)b * kPage + t;
    u4_t ku, vu;
    uint32_t ksb, vsb;
    quant(tok < a.T ? tok : a.T - 1, 1, ku, vu, ksb, vsb);
    const int32_t slot = __shfl(w.slot, kPage + t);
    if ((w.single >> t) & 1u) {
      const int off = slot & (kPage - 1);
      const int64_t page = (int64_t)(slot >> 4) * a.Hkv + h;
      *reinterpret_cast<u4_t *>(kc + page * (kPage * D) + (64 * i + 16 * q + off) * 16) = ku;
      int8_t *vd = vc + page * (kPage * D);
#pragma unroll
      for (int e = 0; e < 16; ++e) vd[i8_v_offset(off, 64 * i + 8 * q + (e & 7) + (e >> 3) * 32)] = (int8_t)unit_byte(vu, e);
      store_scales(page, off, ksb, vsb);
    }
  }
}

// BF16 cache: a scatter copy with the same windows.  Lane (q, t) of wave i holds the two K-page
// rows (2i, q, t) and (2i + 1, q, t) (8 channels each); V pages are staged in LDS.
template <int D>
__global__ __launch_bounds__(D) void kv_write_bf16_kernel(KVQ_WRITE_PARAMS, WriteArgs args) {
  const WriteArgs a = KVQ_WRITE_PLACED(args);
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kPage * D];
  const int b = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, i = threadIdx.x >> 6, q = lane >> 4, t = lane & 15;
  const WriteWindow w = scan_window(a, b, lane);
  const int64_t row_stride = (int64_t)a.Hkv * D;
  uint16_t *kc = static_cast<uint16_t *>(a.kc), *vc = static_cast<uint16_t *>(a.vc);

  if (w.page_t0 >= 0) {
    const int64_t tok = w.page_t0 + t;
    const int64_t page = (int64_t)w.page_blk * a.Hkv + h;
    u4_t ka, kb, va, vb;
    load_row_halves(a.k + tok * row_stride + h * D, i, q, ka, kb);
    load_row_halves(a.v + tok * row_stride + h * D, i, q, va, vb);
    uint16_t *kd = kc + page * (kPage * D);
    *reinterpret_cast<u4_t *>(kd + bf16_k_offset(t, 64 * i + 8 * q)) = ka;
    *reinterpret_cast<u4_t *>(kd + bf16_k_offset(t, 64 * i + 32 + 8 * q)) = kb;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 64 * i + 8 * q + (e & 7) + (e >> 3) * 32;
      const uint32_t wv = e < 8 ? va[(e & 7) >> 1] : vb[(e & 7) >> 1];
      s_v[bf16_v_offset(t, c)] = (uint16_t)((wv >> (16 * (e & 1))) & 0xFFFFu);
    }
    __syncthreads();
    const u4_t *sv = reinterpret_cast<const u4_t *>(s_v);
    u4_t *vd = reinterpret_cast<u4_t *>(vc + page * (kPage * D));
    vd[threadIdx.x] = sv[threadIdx.x];
    vd[threadIdx.x + D] = sv[threadIdx.x + D];
  }

  if (w.single) {
    const int64_t tok = (int64_t)b * kPage + t;
    const int64_t src = (tok < a.T ? tok : a.T - 1) * row_stride + h * D;
    u4_t ka, kb, va, vb;
    load_row_halves(a.k + src, i, q, ka, kb);
    load_row_halves(a.v + src, i, q, va, vb);
    const int32_t slot = __shfl(w.slot, kPage + t);
    if ((w.single >> t) & 1u) {
      const int off = slot & (kPage - 1);
      const int64_t page = (int64_t)(slot >> 4) * a.Hkv + h;
      uint16_t *kd = kc + page * (kPage * D), *vd = vc + page * (kPage * D);
      *reinterpret_cast<u4_t *>(kd + bf16_k_offset(off, 64 * i + 8 * q)) = ka;
      *reinterpret_cast<u4_t *>(kd + bf16_k_offset(off, 64 * i + 32 + 8 * q)) = kb;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 64 * i + 8 * q + (e & 7) + (e >> 3) * 32;
        const uint32_t wv = e < 8 ? va[(e & 7) >> 1] : vb[(e & 7) >> 1];
        vd[bf16_v_offset(off, c)] = (uint16_t)((wv >> (16 * (e & 1))) & 0xFFFFu);
      }
    }
  }
}

// ------------------------------------------------------------------ decode: split partials
//
// Workgroup (split j, KV head h, sequence s) of NW wavefronts.  The split owns pages
// [j*cpp, min((j+1)*cpp, ceil(L/16))); the waves take its pages round-robin, one page per
// unit.  Within a wavefront, lane l = 16*q4 + n16:
//   Q.K   (A = K codes, B = Q):   lane holds scores of head n16, tokens 4*q4 .. 4*q4+3
//   P.V   (A = P',      B = V):   A lane holds P' of head n16 for tokens 4*q4 .. 4*q4+3 (the
//                                 Q.K result layout), as f16 hi and lo parts
//   acc   (P.V result):           lane holds heads 4*q4 .. 4*q4+3 of channel 16*jt + n16
// Per page: Q.K, one softmax update (running max m, sum l, base 2), then P.V; the accumulator
// is rescaled only when some head's maximum grew.  A page's loads are issued as soon as the
// register buffer it lands in has been read out.
// Each split writes an unnormalised partial o = sum_t 2^(x_t - m) v_t with m = max_t x_t,
// x_t = log2(e) * q.k_t / sqrt(D), and l = sum_t 2^(x_t - m).

typedef short s4_t __attribute__((ext_vector_type(4)));

// Register buffers (pages in flight + the page being processed) of the INT8 split kernel.
constexpr int kI8Buffers = 2;

// Max / sum over the four lane rows (lanes n, n+16, n+32, n+48) with the gfx950 row swaps.  The
// max is a comparison, not fmaxf: the swapped values are not known to be canonical floats, so
// fmaxf would first quiet each of them (two more instructions per step).  A NaN score still
// reaches the output through its weight.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a0 = __uint_as_float(a[0]), a1 = __uint_as_float(a[1]);
  x = a0 > a1 ? a0 : a1;
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float b0 = __uint_as_float(b[0]), b1 = __uint_as_float(b[1]);
  return b0 > b1 ? b0 : b1;
}

__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x for x <= 0 (softmax weights); results below 2^-126 may flush to zero, which is far
// below fp32 resolution next to the largest weight (1).
__device__ __forceinline__ float exp2_w(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resource of one page or scale tile: loads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void *base, int64_t index, int bytes,
                                                          int valid_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(base)) + index * bytes, 0,
                                           valid_bytes, 0x00020000);
}

__device__ __forceinline__ u4_t ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Cache page loads.  Where every page is read once per launch (one query token per sequence)
// they carry the non-temporal policy (cache-policy bit 1, `nt` on gfx950): a plain page stream
// over the 32K layer drops from 14.4 to 13.1 us per 71 MB launch with it.  Paths that read a page
// again from L2 or the MALL (several query tokens: several tiles or query chunks per page) keep
// the default policy, which is faster for them.
constexpr int kStreamPolicy = 2;
template <int POL>
__device__ __forceinline__ u4_t ld16_page(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POL));
}
template <int POL>
__device__ __forceinline__ uint32_t ld4_page(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POL);
}

// Q operand (B of Q.K): lane holds head n16 (zero when n16 >= G), channels 32g + 8*q4 + 0..7.
// One buffer resource spans the G query rows of the group; lanes of padding heads fall past
// its end and read zeros, so the loads are unconditional (no divergent branches).
template <int D>
__device__ __forceinline__ void load_q(const DecodeArgs &a, int s, int h, int n16, int q4, u4_t (&qraw)[D / 32]) {
  const uint16_t *rows = a.q + ((int64_t)s * a.Hq + (int64_t)h * a.G) * D;
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(rows), 0, a.G * D * 2, 0x00020000);
  const int off = (n16 * D + 8 * q4) * 2;
#pragma unroll
  for (int g = 0; g < D / 32; ++g) qraw[g] = ld16(r, off, g * kGroup * 2);
}

// ---- quantize-on-write of the step's new token, fused into the split kernel
//
// In a decode step the token at position L - 1 of each sequence is new.  The wavefront that owns
// the sequence's last page (for its KV head) writes the token into that page before it requests
// the page; its own later loads of those bytes follow its stores in order.  Lane l handles
// channels 4l .. 4l + 3 of the K and V rows; lanes with 4l >= D hold zeros and store nothing.

// Requests the new token's K and V rows (4 bf16 per lane); zeros unless `own`.
template <int D>
__device__ __forceinline__ void load_new_rows(const DecodeArgs &a, int s, int h, bool own, int lane, u2_t &kr,
                                              u2_t &vr) {
  const int64_t row = ((int64_t)s * a.Hkv + h) * D;
  const int bytes = own ? 2 * D : 0;
  const uint16_t *kb = own ? a.k_new + row : a.q, *vb = own ? a.v_new + row : a.q;
  kr = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(kb), 0, bytes, 0x00020000),
                                    lane * 8, 0, 0));
  vr = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(vb), 0, bytes, 0x00020000),
                                    lane * 8, 0, 0));
}

// Passes the rows through an empty asm at the top of the write, so that no part of the write
// (which waits for the rows) is hoisted above the branch that selects the writing wave.
__device__ __forceinline__ void pin_rows(u2_t &kr, u2_t &vr) {
  uint32_t k0 = kr[0], k1 = kr[1], v0 = vr[0], v1 = vr[1];
  asm("" : "+v"(k0), "+v"(k1), "+v"(v0), "+v"(v1));
  kr = u2_t{k0, k1};
  vr = u2_t{v0, v1};
}

// INT8 cache: the group maximum is reduced over the 8 lanes of each 32-channel group; scale and
// codes follow the same arithmetic as kv_write (q8_scale, q8_codes), so the bytes are identical.
template <int D>
__device__ __forceinline__ void write_new_i8(const DecodeArgs &a, int64_t page, int t, u2_t kr, u2_t vr, int lane) {
  constexpr int NG = D / kGroup;
  pin_rows(kr, vr);
  const int c0 = 4 * lane;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const uint32_t w0 = which ? vr[0] : kr[0], w1 = which ? vr[1] : kr[1];
    const float x[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    const _Float16 s16 = q8_scale(amax);
    const float sc = (float)s16;
    uint32_t codes;
    q8_codes_div<4>(x, sc, &codes);
    if (c0 < D) {
      int8_t *dst = static_cast<int8_t *>(const_cast<void *>(which ? a.vc : a.kc)) + page * (kPage * D);
      if (which == 0) {
        *reinterpret_cast<uint32_t *>(dst + i8_k_offset(t, c0)) = codes;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i8_v_offset(t, c0 + i)] = (int8_t)((codes >> (8 * i)) & 0xFFu);
      }
      if ((lane & 7) == 0)
        const_cast<uint16_t *>(which ? a.vs : a.ks)[(page * NG + (c0 >> 5)) * kPage + t] =
            __builtin_bit_cast(uint16_t, s16);
    }
  }
}

// Per-head INT8 format: one fp32 scale per (token, head) row.  The row's maximum is reduced over
// the whole wavefront; the scale is amax / 127 (fp32 division), the codes q8_codes(x, scale).
// Returns this lane's 4 codes (one byte each, channels 4 lane .. 4 lane + 3) and the scale.
// BRANCHLESS: the division form (inside the decode kernels).
template <bool BRANCHLESS>
__device__ __forceinline__ uint32_t quant_row_head(uint32_t w0, uint32_t w1, float &scale) {
  const float x[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  scale = amax / 127.0f;
  uint32_t codes;
  if constexpr (BRANCHLESS) q8_codes_div<4>(x, scale, &codes);
  else q8_codes<4>(x, scale, &codes);
  return codes;
}

// Stores one row's codes (K or V in-page order) and its fp32 scale; lanes with 4 lane >= D hold
// no channel and store nothing.
template <int D>
__device__ __forceinline__ void store_row_head(int8_t *page_codes, float *page_scales, int which, int t, int lane,
                                               uint32_t codes, float scale) {
  const int c0 = 4 * lane;
  if (c0 < D) {
    if (which == 0) {
      *reinterpret_cast<uint32_t *>(page_codes + i8_k_offset(t, c0)) = codes;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) page_codes[i8_v_offset(t, c0 + i)] = (int8_t)((codes >> (8 * i)) & 0xFFu);
    }
    if (lane == 0) page_scales[t] = scale;
  }
}

template <int D>
__device__ __forceinline__ void write_new_i8h(const DecodeArgs &a, int64_t page, int t, u2_t kr, u2_t vr, int lane) {
  pin_rows(kr, vr);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const uint32_t w0 = which ? vr[0] : kr[0], w1 = which ? vr[1] : kr[1];
    float scale;
    const uint32_t codes = quant_row_head<true>(w0, w1, scale);
    int8_t *dst = static_cast<int8_t *>(const_cast<void *>(which ? a.vc : a.kc)) + page * (kPage * D);
    float *sc = reinterpret_cast<float *>(const_cast<uint16_t *>(which ? a.vs : a.ks)) + page * kPage;
    store_row_head<D>(dst, sc, which, t, lane, codes, scale);
  }
}

// Per-head INT8 format: one wavefront per (token, KV head, K or V) row; lane l quantizes
// channels 4l .. 4l + 3 (the scale needs the whole row's maximum).
template <int D>
__global__ __launch_bounds__(256) void kv_write_i8h_kernel(KVQ_WRITE_PARAMS, WriteArgs args) {
  const WriteArgs a = KVQ_WRITE_PLACED(args);
  const int lane = threadIdx.x & 63;
  const int64_t rid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rid >= (int64_t)a.T * a.Hkv * 2) return;
  const int which = (int)(rid & 1);
  const int h = (int)((rid >> 1) % a.Hkv);
  const int t = (int)((rid >> 1) / a.Hkv);
  const int32_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.NB * kPage) return;
  const int blk = slot >> 4, off = slot & 15;
  const uint16_t *src = (which ? a.v : a.k) + ((int64_t)t * a.Hkv + h) * D;
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(src), 0, D * 2, 0x00020000);
  const u2_t w = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8, 0, 0));
  float scale;
  const uint32_t codes = quant_row_head<false>(w[0], w[1], scale);
  const int64_t page = (int64_t)blk * a.Hkv + h;
  int8_t *dst = static_cast<int8_t *>(which ? a.vc : a.kc) + page * (kPage * D);
  float *sc = reinterpret_cast<float *>(which ? a.vs : a.ks) + page * kPage;
  store_row_head<D>(dst, sc, which, off, lane, codes, scale);
}

// BF16 cache: a copy of the two rows into the page.
template <int D>
__device__ __forceinline__ void write_new_bf16(const DecodeArgs &a, int64_t page, int t, u2_t kr, u2_t vr, int lane) {
  pin_rows(kr, vr);
  const int c0 = 4 * lane;
  if (c0 < D) {
    uint16_t *kd = static_cast<uint16_t *>(const_cast<void *>(a.kc)) + page * (kPage * D);
    uint16_t *vd = static_cast<uint16_t *>(const_cast<void *>(a.vc)) + page * (kPage * D);
    *reinterpret_cast<u2_t *>(kd + bf16_k_offset(t, c0)) = kr;
    const uint32_t v01 = vr[0], v23 = vr[1];
    vd[bf16_v_offset(t, c0)] = (uint16_t)(v01 & 0xFFFFu);
    vd[bf16_v_offset(t, c0 + 1)] = (uint16_t)(v01 >> 16);
    vd[bf16_v_offset(t, c0 + 2)] = (uint16_t)(v23 & 0xFFFFu);
    vd[bf16_v_offset(t, c0 + 3)] = (uint16_t)(v23 >> 16);
  }
}

// Q operand for several query tokens: MFMA row r = 16 * rt + n16 of KV head h is the pair
// (query token c0 + r / G, head h * G + r % G) of the workgroup's chunk (query tokens c0 ..
// c0 + n_here - 1); rows past n_here * G read zeros.
template <int D>
__device__ __forceinline__ void load_q_mq(const DecodeArgs &a, int s, int h, int rt, int c0, int n_here, int n16,
                                          int q4, u4_t (&qraw)[D / 32]) {
  const uint16_t *base = a.q + (int64_t)s * a.nq * a.Hq * D;
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, a.nq * a.Hq * D * 2, 0x00020000);
  const int row = 16 * rt + n16;
  const int i = row / a.G, g = row - i * a.G;  // query token c0 + i of the chunk, head h * G + g
  const int off = row < n_here * a.G ? ((((c0 + i) * a.Hq + h * a.G + g) * D) + 8 * q4) * 2 : 0x40000000;
#pragma unroll
  for (int gg = 0; gg < D / 32; ++gg) qraw[gg] = ld16(r, off, gg * kGroup * 2);
}

// Merge scratch of one wave (floats): its accumulator tiles as [tile][lane][4], then m[16]
// and l[16].
template <int D>
constexpr int merge_stride() { return (D / 16) * 256 + 32; }

// Writes the partial of this wavefront (NW == 1) or of the whole workgroup (NW > 1: an LDS
// merge; `merge` holds NW regions of merge_stride<D>() floats).  Every wave stores its
// accumulator tiles as they sit in its registers; wave w then combines tiles w, w + NW, ...
// of all waves for its own lanes' rows, each wave's rows weighted by 2^(m_w - M).
// Several row tiles per workgroup (RTW > 1): waves w, w + RTW, ... hold the same tile (rl = w % RTW)
// for different pages and merge among themselves.
template <int D, int NW, bool MQ = false, int RTW = 1>
__device__ __forceinline__ void write_partial(const DecodeArgs &a, int s, int h, int j, int wave, int n16, int q4,
                                              float m_run, float l_run, const f4_t (&acc)[D / 16], float *merge,
                                              int rt = 0, int c0 = 0, int n_here = 1) {
  constexpr int NT = D / 16;
  constexpr int ST = merge_stride<D>();
  constexpr int NWP = NW / RTW;  // waves per row tile
  static_assert(NW % RTW == 0 && NT % NWP == 0, "waves must split evenly over row tiles and output tiles");
  const int rl = wave % RTW, pw = wave / RTW;
  const int G = a.G;
  const int lane = q4 * 16 + n16;
  l_run = rows_sum(l_run);
  const int64_t row0 = ((int64_t)s * a.Hq + (int64_t)h * G) * a.NS + j;  // partial of head h*G + 0
  static_assert(!(MQ && NW == 1), "several query tokens use the LDS merge path");
  if constexpr (MQ && NWP == 1) {
    // One wave per row tile: the tile's partial sits in this wave's registers, no LDS merge.
    // Tile row r is (query token c0 + (16 rt + r) / G, head h G + (16 rt + r) % G); rows past the
    // chunk's n_here * G real rows map past the end of the resources and their stores are dropped.
    const int64_t seq0 = (int64_t)s * a.nq * a.Hq * a.NS;  // first partial row of the sequence
    const int rows_valid = a.nq * a.Hq * a.NS;
    // (an opaque copy of G: the division's constants are recomputed here, not kept live from the
    // caller's prologue)
    int Gd = G;
    asm volatile("" : "+s"(Gd));
    auto row_offset = [&](int r) -> int {
      const int row = 16 * rt + r;
      const int t = row / Gd, g = row - t * Gd;
      return row < n_here * G ? ((c0 + t) * a.Hq + h * G + g) * a.NS + j : rows_valid;
    };
    if (q4 == 0) {  // (m, l) of row n16 (the same in the row's 4 lanes)
      const auto rml = __builtin_amdgcn_make_buffer_rsrc(a.ml + seq0, 0, rows_valid * 8, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2_t, make_float2(m_run, l_run)), rml,
                                            row_offset(n16) * 8, 0, 0);
    }
    const auto ro = __builtin_amdgcn_make_buffer_rsrc(a.o_part + seq0 * D, 0, rows_valid * D * 4, 0x00020000);
    int row_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) row_off[i] = row_offset(4 * q4 + i);
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[jt][i]), ro, (row_off[i] * D + 16 * jt + n16) * 4, 0, 0);
  } else if constexpr (NW == 1) {
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 4 * q4 + i;
        if (hh < G) a.o_part[(row0 + (int64_t)hh * a.NS) * D + 16 * jt + n16] = acc[jt][i];
      }
    if (q4 == 0 && n16 < G) a.ml[row0 + (int64_t)n16 * a.NS] = make_float2(m_run, l_run);
  } else {
    float *mine = merge + wave * ST;
    const int rows_here = MQ ? min(n_here * G - 16 * rt, 16) : G;  // real rows of this tile
    if (4 * q4 < rows_here) {  // lanes that hold a real row
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) *reinterpret_cast<f4_t *>(mine + (jt * 64 + lane) * 4) = acc[jt];
    }
    if (q4 == 0) {
      mine[NT * 256 + n16] = m_run;
      mine[NT * 256 + 16 + n16] = l_run;
    }
    __syncthreads();
    // Every lane computes; lanes of padding heads (4 q4 + i >= G) read unused LDS and their stores
    // fall past the end of the resources below (rows of heads 0 .. G-1 only), so no branches.
    // weights of every wave for this lane's rows (heads 4 q4 .. 4 q4 + 3)
    f4_t mw[NWP], wt[NWP];
    f4_t M = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int w = 0; w < NWP; ++w) {
      mw[w] = *reinterpret_cast<const f4_t *>(merge + (rl + w * RTW) * ST + NT * 256 + 4 * q4);
#pragma unroll
      for (int i = 0; i < 4; ++i) M[i] = fmaxf(M[i], mw[w][i]);
    }
    f4_t Lsum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < NWP; ++w) {
      const f4_t lw = *reinterpret_cast<const f4_t *>(merge + (rl + w * RTW) * ST + NT * 256 + 16 + 4 * q4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wt[w][i] = (mw[w][i] == -INFINITY) ? 0.0f : exp2_w(mw[w][i] - M[i]);  // waves without pages: 0
        Lsum[i] = fmaf(wt[w][i], lw[i], Lsum[i]);
      }
    }
    // row_off[i]: offset (in partial rows) of this lane's row 4 q4 + i from the resources' base;
    // rows past the end of the resources are dropped by the bounds check
    int row_off[4];
    int rows_valid;
    const float2 *ml_base;
    const float *o_base;
    if constexpr (MQ) {
      // tile row 16 rt + r is (query token c0 + (16 rt + r) / G, head h G + (16 rt + r) % G)
      const int64_t seq0 = (int64_t)s * a.nq * a.Hq * a.NS;  // first partial row of the sequence
      rows_valid = a.nq * a.Hq * a.NS;
      ml_base = a.ml + seq0;
      o_base = a.o_part + seq0 * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * rt + 4 * q4 + i;
        const int t = row / G, g = row - t * G;
        row_off[i] = row < n_here * G ? ((c0 + t) * a.Hq + h * G + g) * a.NS + j : rows_valid;
      }
    } else {
      rows_valid = (G - 1) * a.NS + 1;  // rows from head 0 through head G - 1 of this split
      ml_base = a.ml + row0;
      o_base = a.o_part + row0 * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) row_off[i] = (4 * q4 + i) * a.NS;
    }
    if (pw == 0 && n16 == 0) {
      const auto rml = __builtin_amdgcn_make_buffer_rsrc(const_cast<float2 *>(ml_base), 0, rows_valid * 8, 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(u2_t, make_float2(M[i], Lsum[i])), rml, row_off[i] * 8, 0, 0);
    }
    const auto ro = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(o_base), 0, rows_valid * D * 4, 0x00020000);
    f4_t o[NT / NWP];
#pragma unroll
    for (int t = 0; t < NT / NWP; ++t) {  // every LDS read is issued before the first store
      const int jt = pw + t * NWP;
      o[t] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < NWP; ++w) {
        const f4_t v = *reinterpret_cast<const f4_t *>(merge + (rl + w * RTW) * ST + (jt * 64 + lane) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i] = fmaf(wt[w][i], v[i], o[t][i]);
      }
    }
#pragma unroll
    for (int t = 0; t < NT / NWP; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[t][i]), ro,
                                              (row_off[i] * D + 16 * (pw + t * NWP) + n16) * 4, 0, 0);
  }
}

// s_waitcnt with only the vector-memory count set (expcnt and lgkmcnt at their maxima: no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The decode split kernels take the values that place a workgroup and its first memory requests
// (block table, context lengths, split and head counts, pages per split, table width, row groups,
// query chunks) as leading scalar arguments, ahead of the argument block: the hardware preloads
// them into scalar registers at launch, and the rest of the block is read during the first round
// trip instead of before it.  placed() makes the kernel's working copy of the block use them.
#define KVQ_PLACEMENT_PARAMS                                                                              \
  const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens, int num_splits,     \
      int num_kv_heads, int pages_per_split, int max_blocks, int row_groups, int chunks, int qchunk, int nq
__device__ __forceinline__ DecodeArgs placed(const DecodeArgs &args, int num_splits, int num_kv_heads,
                                             int pages_per_split, int max_blocks, int row_groups, int chunks,
                                             int qchunk, int nq) {
  DecodeArgs a = args;
  a.NS = num_splits;
  a.Hkv = num_kv_heads;
  a.cpp = pages_per_split;
  a.max_blocks = max_blocks;
  a.row_groups = row_groups;
  a.chunks = chunks;
  a.qchunk = qchunk;
  a.nq = nq;
  return a;
}
#define KVQ_PLACED(args) \
  placed(args, num_splits, num_kv_heads, pages_per_split, max_blocks, row_groups, chunks, qchunk, nq)

// ---- INT8 cache: 1-page units in a ring of register buffers, f16 MFMA for both products
//
// A wave owns pages p0 + wave + k * NW (k = 0, 1, ...) of its split (several query tokens with
// RTW row tiles per workgroup: pages p0 + wave / RTW + k * NW / RTW, for tile wave % RTW).  Page k lands in register
// buffer k % NBUF; the page is requested as soon as its buffer has been read out, so while the
// wave works on one page the next NBUF - 1 are in flight.  Q and the first page are requested
// before anything else; the other buffers fill once Q has arrived.
template <int D, int NW, int MQR, int FMT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_i8_kernel(KVQ_PLACEMENT_PARAMS, DecodeArgs args) {
  const DecodeArgs a = KVQ_PLACED(args);
  constexpr bool MQ = MQR > 0;        // several query tokens: rows are (query token, head) pairs
  constexpr int RTW = MQ ? MQR : 1;   // row tiles per workgroup (MQ)
  constexpr int NWP = NW / RTW;       // waves that split the pages of one row tile
  static_assert(NW % RTW == 0, "row tiles must split the waves evenly");
  constexpr bool HEADSC = FMT == 1;   // per-head format: one fp32 scale per token (else q8_0)
  constexpr bool IQK = FMT == 2;      // q8_0 with integer Q.K: Q quantized per 32 values like the cache
  constexpr int NG = D / kGroup;      // scale groups
  constexpr int NT = D / 16;          // output tiles
  constexpr int NL = D / 64;          // 16-byte code loads per lane per page
  constexpr int PAGE_B = kPage * D;   // bytes of one code page
  constexpr int SCALE_B = HEADSC ? kPage * 4 : kPage * NG * 2;  // bytes of one scale tile
  constexpr int NBUF = kI8Buffers;
  // page loads: non-temporal when each page is read once (one row tile); the tiles of a
  // multi-tile workgroup read each page once each, the second time from L2
  constexpr int POL = RTW > 1 ? 0 : kStreamPolicy;
  __shared__ __attribute__((aligned(16))) uint32_t s_sc[NW][2][SCALE_B / 4];  // K, V scale tiles (group-major)
  __shared__ __attribute__((aligned(16))) h8_t s_q[RTW][NG][64];              // Q operand fragments per row tile
  __shared__ __attribute__((aligned(16))) float s_alpha[NW][16];              // rescale factors, per head
  extern __shared__ float s_merge[];                                          // [NW][G*D + 32] (dynamic)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: keeps page math scalar
  const int rl = wave % RTW, pw = wave / RTW;  // row tile within the workgroup, page-wave index
  const int n16 = lane & 15, q4 = lane >> 4;
  const int j = blockIdx.x % a.NS;
  // (MQ: the workgroup's group of RTW 16-row tiles of (query token, head) pairs, between split and
  // KV head; this wave's tile is rt)
  const int rg = MQ ? (blockIdx.x / a.NS) % a.row_groups : 0;
  const int rt = rg * RTW + rl;
  const int h = (blockIdx.x / (a.NS * (MQ ? a.row_groups : 1))) % a.Hkv;
  // MQ: the query chunk (tokens c0 .. c0 + n_here - 1 of the sequence's nq), between KV head and
  // sequence; it attends over the keys up to its last query token
  const int c = MQ ? (blockIdx.x / (a.NS * a.row_groups * a.Hkv)) % a.chunks : 0;
  const int s = blockIdx.x / (a.NS * (MQ ? a.row_groups * a.chunks : 1) * a.Hkv);
  const int c0 = c * (MQ ? a.qchunk : 1);
  const int n_here = MQ ? min(a.qchunk, a.nq - c0) : 1;
  const int p0 = j * a.cpp;
  const int32_t *btrow = block_tables + (int64_t)s * a.max_blocks;
  const int voff = lane * 16;  // byte offset of this lane's 16-byte fragment in each KiB of a page

  // Block id of page k of the wave: a scalar load (the block table is only read here), issued
  // one page ahead of its use so that its latency hides behind a page's work.  The index is
  // clamped to the table row, not to the context, so the first ids are requested together with
  // the context length (one round trip before the first page request, not two); ids of pages past
  // the split are never used to read memory (their loads have size-0 resources).
  auto block_of = [&](int k) -> int { return btrow[min(p0 + pw + k * NWP, a.max_blocks - 1)]; };
  auto page_of = [&](int blk) -> int64_t { return (int64_t)min(max(blk, 0), a.NB - 1) * a.Hkv + h; };
  int blk[NBUF];
#pragma unroll
  for (int b = 0; b < NBUF; ++b) blk[b] = block_of(b);
  // Q and the step's new token (every wave requests the token's rows; the owning wave, known once
  // the length has arrived, writes it) are requested in the same round trip.
  u4_t qraw[NG];
  if constexpr (MQ) load_q_mq<D>(a, s, h, rt, c0, n_here, n16, q4, qraw);
  else load_q<D>(a, s, h, n16, q4, qraw);
  u2_t knew, vnew;
  load_new_rows<D>(a, s, h, !MQ && a.k_new != nullptr, lane, knew, vnew);

  const int L_raw = context_lens[s];
  const int L_full = max(0, min(L_raw, a.max_context_len));
  const int L = MQ ? max(0, L_full - a.nq + c0 + n_here) : L_full;
  const int P = (L + kPage - 1) / kPage;
  const int p1 = min(p0 + a.cpp, P);
  if (p0 >= p1) {  // empty split: nothing written, the merge skips it
    // The prologue's loads and the arguments the page requests need are used on this path too, so
    // the compiler issues them all before the branch (one round trip before the first page
    // request) instead of sinking them into the other path behind further waits.
    asm volatile("" ::"s"(blk[0]), "s"(blk[NBUF - 1]), "s"(a.kc), "s"(a.vc), "s"(a.ks), "s"(a.vs), "s"(a.NB),
                 "v"(qraw[0][0]), "v"(knew[0]));
    return;
  }
  const int n_units = p1 - p0;

  // ---- register buffers: K / V codes and the page's K / V scale tiles (one dword per lane).
  // Past the end of the split the resources have size 0: the loads return zeros without
  // touching memory, so they are issued unconditionally (no divergent branch, no wait merge).
  u4_t kb[NBUF][NL], vb[NBUF][NL];
  // scale registers: q8_0 one dword of the tile per lane (restaged through LDS); per-head the
  // fp32 scales of the lane's 4 tokens
  using scale_reg_t = typename std::conditional<HEADSC, u4_t, uint32_t>::type;
  scale_reg_t ksb[NBUF], vsb[NBUF];
  auto load_scales = [&](const void *plane, int64_t page, bool ok) -> scale_reg_t {
    const auto r = page_rsrc(plane, page, SCALE_B, ok ? SCALE_B : 0);
    if constexpr (HEADSC) return ld16_page<POL>(r, q4 * 16, 0);
    else return ld4_page<POL>(r, lane * 4, 0);
  };
  auto issue_k = [&](int b, int k, int blk) {
    const bool ok = pw + k * NWP < n_units;
    const int64_t page = page_of(blk);
    const auto r = page_rsrc(a.kc, page, PAGE_B, ok ? PAGE_B : 0);
#pragma unroll
    for (int i = 0; i < NL; ++i) kb[b][i] = ld16_page<POL>(r, voff, 1024 * i);
    ksb[b] = load_scales(a.ks, page, ok);
  };
  auto issue_v = [&](int b, int k, int blk) {
    const bool ok = pw + k * NWP < n_units;
    const int64_t page = page_of(blk);
    const auto r = page_rsrc(a.vc, page, PAGE_B, ok ? PAGE_B : 0);
#pragma unroll
    for (int i = 0; i < NL; ++i) vb[b][i] = ld16_page<POL>(r, voff, 1024 * i);
    vsb[b] = load_scales(a.vs, page, ok);
  };

  // The wave that holds the sequence's last page writes the step's new token into it (its local
  // page index k_last) before it requests that page.  A length above max_context_len (outside the
  // contract) writes nothing.  Ordering: vmcnt counts this wave's stores until the memory system
  // has acknowledged them (then a later load of the same bytes, which misses the write-through L1,
  // reads them back), and it retires in issue order; so before requesting page k_last the owner
  // waits until at most the loads issued after its stores are outstanding (the waits below).
  bool own_new = !MQ && a.k_new != nullptr && L_raw <= a.max_context_len && p1 == P && wave == (n_units - 1) % NW;
  const int blk_last = own_new ? btrow[P - 1] : 0;  // (only the owner waits for it)
  own_new = own_new && blk_last >= 0 && blk_last < a.NB;
  const int k_last = (n_units - 1) / NWP;
  // MQ: the lane's row sees keys 0 .. L - nq + token (causal among the query tokens)
  int L_row = L;
  if constexpr (MQ) L_row = L_full - a.nq + c0 + (16 * rt + n16) / a.G + 1;
  const int L_min = L_full - a.nq + c0 + 1;  // (MQ) the chunk's first query token's limit, the smallest
  __builtin_amdgcn_sched_barrier(0);
  const int64_t page_new = (int64_t)blk_last * a.Hkv + h;
  const int t_new = (L - 1) & (kPage - 1);
  auto write_new = [&] {
    if constexpr (HEADSC) write_new_i8h<D>(a, page_new, t_new, knew, vnew, lane);
    else write_new_i8<D>(a, page_new, t_new, knew, vnew, lane);
  };
  if (own_new && k_last == 0) {
    write_new();
    wait_vmcnt<0>();  // the stores are the youngest memory operations
  }
  issue_k(0, 0, blk[0]);
  __builtin_amdgcn_sched_barrier(0);
  issue_v(0, 0, blk[0]);
  __builtin_amdgcn_sched_barrier(0);

  // Q: bf16 rescaled by 2^shift per head so that max |q| lies in [2^14, 2^15): exact in f16.
  // Every wave derives the per-head shift; wave 0 stores the operand into LDS ([group][lane]
  // 16-byte fragments) for all waves.
  int shift = 0;
  {
    float qmax = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(qraw[g][e])), fabsf(bf16_hi(qraw[g][e]))));
    qmax = rows_max(qmax);
    if (qmax > 0.0f) {
      int e2;
      frexpf(qmax, &e2);
      shift = 15 - e2;
    }
    if (pw == 0) {  // (one wave per row tile)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        h8_t qg;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qg[2 * e] = (_Float16)ldexpf(bf16_lo(qraw[g][e]), shift);
          qg[2 * e + 1] = (_Float16)ldexpf(bf16_hi(qraw[g][e]), shift);
        }
        s_q[rl][g][lane] = qg;
      }
    }
    // LDS-only fences: __syncthreads would also wait for the page loads in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
  const float cmul = ldexpf(kLog2e / sqrtf((float)D), IQK ? 0 : -shift);
  // integer Q.K: every wave quantizes its Q rows with the cache's q8_0 rule (fp16 scale of the
  // group's amax / 127, codes against the stored scale): qi[g] holds the lane's 8 codes of group g
  // (the B operand of v_mfma_i32_16x16x32_i8), sq[g] the row's scale for group g
  uint64_t qi[IQK ? NG : 1];
  float sq[IQK ? NG : 1];
  if constexpr (IQK) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_lo(qraw[g][e]);
        x[2 * e + 1] = bf16_hi(qraw[g][e]);
      }
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
      amax = rows_max(amax);  // the group's 32 values sit in the 4 lanes of the row
      const float sc16 = (float)q8_scale(amax);
      uint32_t lohi[2];
      q8_codes_div<8>(x, sc16, lohi);
      const uint32_t lo = lohi[0], hi = lohi[1];
      qi[g] = ((uint64_t)hi << 32) | lo;
      sq[g] = sc16;
    }
  }
  if (own_new && k_last != 0) {
    write_new();
    if (k_last < NBUF) wait_vmcnt<0>();  // page k_last is requested right below
  }
#pragma unroll
  for (int b = 1; b < NBUF; ++b) {
    issue_k(b, b, blk[b]);
    issue_v(b, b, blk[b]);
    __builtin_amdgcn_sched_barrier(0);
  }
  int blk_next = block_of(NBUF);

  float m_run = -INFINITY, l_run = 0.0f;
  // per-head format: acc holds the value sum times 2^(kPvBias - r_run), r_run the largest V-scale
  // exponent seen so far: P' = p * s_v * 2^(kPvBias - r_run) stays below 2^kPvBias (f16 range,
  // whatever the scales), and tokens whose scale is up to about 2^kPvBias below the largest one
  // still have P' in f16's normal range (below it hi and lo keep only absolute precision)
  constexpr int kPvBias = 14;
  int r_run = -1000;
  f4_t acc[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) acc[jt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // the Q operand stays in registers for the whole split
  h8_t qop[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) qop[g] = s_q[rl][g][lane];
  // Scale tiles are restaged token-quad-major ([q4][group][4 tokens]) so that a lane reads the
  // scales of its 4 tokens for all groups with 8*NG contiguous bytes.  Tile dword l (group-major
  // [group][token]) holds group l / 8, tokens 2 (l % 8) and 2 (l % 8) + 1.
  const int st_dw = (((lane & 7) >> 1) * NG + (lane >> 3)) * 2 + (lane & 1);  // restaged dword of dword l
  auto stage = [&](int which, uint32_t w) {
    if (lane < kPage * NG * 2 / 4) s_sc[wave][which][st_dw] = w;
  };
  auto scales = [&](int which, u2_t (&out)[NG]) {
    const u4_t *src = reinterpret_cast<const u4_t *>(&s_sc[wave][which][q4 * NG * 2]);
#pragma unroll
    for (int i = 0; i < NG / 2; ++i) {
      const u4_t w = src[i];
      out[2 * i] = u2_t{w[0], w[1]};
      out[2 * i + 1] = u2_t{w[2], w[3]};
    }
  };

  // One page from buffer b: Q.K^T, one online-softmax update, P.V.
  auto process = [&](int b, int k) {
    const int u = pw + k * NWP;  // (past the split's last page: no valid token)
    const int lim = u < n_units ? min(L - (p0 + u) * kPage, kPage) : 0;  // valid tokens of the page
    f4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (HEADSC) {
      // ---- Q.K^T, per-head format: the groups' MFMAs accumulate in two chains, then each token's
      // fp32 scale (tokens past the context may carry any scale: their scores are masked below)
      f4_t c0 = {0.0f, 0.0f, 0.0f, 0.0f}, c1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const h8_t kop = i8x8_to_h8(kb[b][g >> 1][(g & 1) * 2], kb[b][g >> 1][(g & 1) * 2 + 1]);
        if (g & 1) c1 = mfma_f16(kop, qop[g], c1);
        else c0 = mfma_f16(kop, qop[g], c0);
      }
      const u4_t ks4 = ksb[b];
      const uint32_t k0 = ks4[0], k1 = ks4[1], k2 = ks4[2], k3 = ks4[3];
      sc[0] = (c0[0] + c1[0]) * __uint_as_float(k0);
      sc[1] = (c0[1] + c1[1]) * __uint_as_float(k1);
      sc[2] = (c0[2] + c1[2]) * __uint_as_float(k2);
      sc[3] = (c0[3] + c1[3]) * __uint_as_float(k3);
    } else {
    stage(0, ksb[b]);
    u2_t ksc[NG];
    scales(0, ksc);
    // ---- Q.K^T: one MFMA per 32-channel group, then the group's fp16 scale
    // one MFMA per group; the scale step of group g runs after group g + 1's MFMA is issued
    auto qk_group = [&](int g) -> f4_t {
      if constexpr (IQK) {  // exact int32 dot products of the codes, as fp32 times the Q scale
        const uint32_t d0 = kb[b][g >> 1][(g & 1) * 2], d1 = kb[b][g >> 1][(g & 1) * 2 + 1];
        const auto ci = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)(((uint64_t)d1 << 32) | d0), (long)qi[g],
                                                              v4i_t{0, 0, 0, 0}, 0, 0, 0);
        return f4_t{(float)ci[0] * sq[g], (float)ci[1] * sq[g], (float)ci[2] * sq[g], (float)ci[3] * sq[g]};
      } else {
        return mfma_f16(i8x8_to_h8(kb[b][g >> 1][(g & 1) * 2], kb[b][g >> 1][(g & 1) * 2 + 1]), qop[g],
                        f4_t{0.0f, 0.0f, 0.0f, 0.0f});
      }
    };
    auto scale_group = [&](int g, const f4_t &c) {
      const u2_t sw = ksc[g];
      sc[0] = fma_h16lo(sw[0], c[0], sc[0]);
      sc[1] = fma_h16hi(sw[0], c[1], sc[1]);
      sc[2] = fma_h16lo(sw[1], c[2], sc[2]);
      sc[3] = fma_h16hi(sw[1], c[3], sc[3]);
      pin4(sc);  // keeps the scale step here (else every group's result stays live)
    };
    f4_t c_prev = qk_group(0);
#pragma unroll
    for (int g = 1; g < NG; ++g) {
      const f4_t c = qk_group(g);
      scale_group(g - 1, c_prev);
      c_prev = c;
      __builtin_amdgcn_sched_barrier(0);
    }
    scale_group(NG - 1, c_prev);
    }
    // ---- online softmax over the page's 16 tokens (base 2).  Padding heads (Q = 0) get finite
    // scores; their rows are never written out.
    float x[4];
    int lim_row = lim;  // valid tokens of the page for this lane's row
    if constexpr (MQ) lim_row = u < n_units ? min(max(L_row - (p0 + u) * kPage, 0), kPage) : 0;
    if (MQ && u < n_units && (p0 + u + 1) * kPage <= L_min) {  // (uniform) every row sees the whole page
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = sc[i] * cmul;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (4 * q4 + i < lim_row) ? sc[i] * cmul : -INFINITY;
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = rows_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = (m_new == m_run) ? 1.0f : exp2_w(m_run - m_use);
    const bool grew = alpha != 1.0f && m_run != -INFINITY;  // (the first update finds acc = 0)
    float p[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2_w(x[i] - m_use);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(grew)) {  // some head's maximum grew: rescale its accumulator rows
      if (q4 == 0) s_alpha[wave][n16] = alpha;
      const f4_t ar = *reinterpret_cast<const f4_t *>(&s_alpha[wave][4 * q4]);  // heads 4*q4 .. +3
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) acc[jt] *= ar;
    }
    const int nv = min(max(lim - 4 * q4, 0), 4);  // valid tokens among the lane's 4
    if constexpr (HEADSC) {
      // ---- P.V, per-head format: P' = p * s_v * 2^(kPvBias - r_run) per token (once per page), f16 hi + lo
      // packed along K as below.  Scales of tokens past the context are masked to 0.
      const u4_t vs4 = vsb[b];
      const uint32_t w0 = vs4[0], w1 = vs4[1], w2 = vs4[2], w3 = vs4[3];
      const float sv[4] = {nv > 0 ? __uint_as_float(w0) : 0.0f, nv > 1 ? __uint_as_float(w1) : 0.0f,
                           nv > 2 ? __uint_as_float(w2) : 0.0f, nv > 3 ? __uint_as_float(w3) : 0.0f};
      // the page's largest V scale (the same in every lane) sets the exponent
      const float smax = rows_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      const int e_page = smax > 0.0f ? __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(smax)) : r_run;
      if (e_page > r_run) {  // (uniform) exact power-of-two rescale of the accumulator
        const float beta = ldexpf(1.0f, r_run - e_page);
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) acc[jt] *= beta;
        r_run = e_page;
      }
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = p[i] * ldexpf(sv[i], kPvBias - r_run);
      const h2_t hi01 = {(_Float16)pv[0], (_Float16)pv[1]}, hi23 = {(_Float16)pv[2], (_Float16)pv[3]};
      const h2_t lo01 = {(_Float16)(pv[0] - (float)hi01[0]), (_Float16)(pv[1] - (float)hi01[1])};
      const h2_t lo23 = {(_Float16)(pv[2] - (float)hi23[0]), (_Float16)(pv[3] - (float)hi23[1])};
      const h8_t pp = __builtin_bit_cast(h8_t, u4_t{__builtin_bit_cast(uint32_t, hi01), __builtin_bit_cast(uint32_t, hi23),
                                                   __builtin_bit_cast(uint32_t, lo01), __builtin_bit_cast(uint32_t, lo23)});
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        uint32_t v0, v1;
        i8x4_to_f16(vb[b][jt >> 2][jt & 3], v0, v1);
        acc[jt] = mfma_f16(pp, __builtin_bit_cast(h8_t, u4_t{v0, v1, v0, v1}), acc[jt]);
      }
    } else {
    // ---- P.V: P' = p * s_v per (token, group) as f16 hi + lo, times exact f16 V codes.  V scales
    // of tokens past the context are masked to 0 (their codes and scales may be stale).
    stage(1, vsb[b]);
    u2_t vsc[NG];
    scales(1, vsc);
    const u2_t msk = {nv >= 2 ? 0xFFFFFFFFu : (nv == 1 ? 0xFFFFu : 0u), nv >= 4 ? 0xFFFFFFFFu : (nv == 3 ? 0xFFFFu : 0u)};
    // One 16x16x32 MFMA per output tile covers both parts of P': its 32 K-slots are, per lane,
    // (hi of tokens 4 q4 .. 4 q4 + 3, lo of the same tokens), and the V operand holds the lane's
    // 4 codes twice.
    // P' = p * s_v as f16 hi + lo with packed f16 arithmetic, two tokens per instruction:
    // p = ph + pl (f16 hi / lo of p, once per page), hi = f16(ph * s), lo = f16(pl * s + r) with
    // r = ph * s - hi exact (a fused multiply-add); hi + lo is within about 2^-21 of p * s.
    const h2_t ph01 = {(_Float16)p[0], (_Float16)p[1]}, ph23 = {(_Float16)p[2], (_Float16)p[3]};
    const h2_t pl01 = {(_Float16)(p[0] - (float)ph01[0]), (_Float16)(p[1] - (float)ph01[1])};
    const h2_t pl23 = {(_Float16)(p[2] - (float)ph23[0]), (_Float16)(p[3] - (float)ph23[1])};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const u2_t sv = vsc[g] & msk;
      // (through scalars: a bit cast of a vector element subscript reads the wrong element)
      const uint32_t w01 = sv[0], w23 = sv[1];
      const h2_t s01 = __builtin_bit_cast(h2_t, w01), s23 = __builtin_bit_cast(h2_t, w23);
      const h2_t hi01 = ph01 * s01, hi23 = ph23 * s23;
      const h2_t lo01 = __builtin_elementwise_fma(pl01, s01, __builtin_elementwise_fma(ph01, s01, -hi01));
      const h2_t lo23 = __builtin_elementwise_fma(pl23, s23, __builtin_elementwise_fma(ph23, s23, -hi23));
      const h8_t pp = __builtin_bit_cast(h8_t, u4_t{__builtin_bit_cast(uint32_t, hi01), __builtin_bit_cast(uint32_t, hi23),
                                                   __builtin_bit_cast(uint32_t, lo01), __builtin_bit_cast(uint32_t, lo23)});
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int jt = 2 * g + jj;
        uint32_t v0, v1;
        i8x4_to_f16(vb[b][jt >> 2][jt & 3], v0, v1);
        acc[jt] = mfma_f16(pp, __builtin_bit_cast(h8_t, u4_t{v0, v1, v0, v1}), acc[jt]);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep each group's temporaries short-lived
    }
    }
  };

  // A uniform trip count and no early exit: pages past the split's end read zeros and are
  // fully masked (p = 0), which keeps the in-flight buffers in fixed registers across the loop.
  const int my_units = pw < n_units ? (n_units - pw + NWP - 1) / NWP : 0;
  // Loads per page (K and V codes, K and V scale tiles).  When page k_last (>= NBUF) is about to be
  // requested, only the NBUF - 1 pages requested after it may still be outstanding: everything
  // older, the owner's stores included (they were issued before page 1), has completed.
  constexpr int kPageLoads = 2 * (NL + 1);
  for (int k = 0; k < my_units; k += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      process(b, k + b);
      if (own_new && k + b + NBUF == k_last) wait_vmcnt<kPageLoads * (NBUF - 1)>();
      issue_k(b, k + b + NBUF, blk_next);
      issue_v(b, k + b + NBUF, blk_next);
      __builtin_amdgcn_sched_barrier(0);
      blk_next = block_of(k + b + NBUF + 1);
    }
  }
  if constexpr (HEADSC) {  // back to the true value sum: acc * 2^(r_run - kPvBias)
    const float f = ldexpf(1.0f, r_run - kPvBias);
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) acc[jt] *= f;
  }
  write_partial<D, NW, MQ, RTW>(a, s, h, j, wave, n16, q4, m_run, l_run, acc, s_merge, rt, c0, n_here);
}

// ---- INT8 cache (q8_0), several query tokens in 4 row tiles: the waves walk the pages together
//
// Workgroup (split, KV head, query chunk, sequence) of 4 waves, one 16-row tile of (query token,
// head) pairs each: the rows, grid and partials of decode_split_i8_kernel<D, 4, 4, 0>.  Instead
// of every wave loading and converting every page, the workgroup loads each page once: thread t
// takes the page's 16-byte code chunks t, t + 256, ... (K chunks first, then V; D / 128 per
// thread), converts them to the f16 MFMA fragments and stores them in LDS, and waves 0 and 1 stage
// the K and V scale tiles.  After one barrier every wave reads the fragments of all groups from
// LDS and runs the decode kernel's page step on its own tile (Q.K per group and fp16 scale,
// online softmax, P' = p * s_v as f16 hi + lo, P.V as two K = 16 products, hi then lo, on one
// read of each V operand, which LDS holds once).  LDS holds two pages, so the stores of page
// k + 1 never meet the reads of page k - 1; each thread holds a quarter or an eighth of a page in
// registers, so NBUF pages are in flight at little register cost.  Two forms, both with 2 pages in
// flight:
// - PG = 2 page groups of 4 waves, registers uncapped (one chunk of query tokens, e.g. a decode
//   of 6 to 10 tokens): group g takes pages 2 i + g of the split, each group with its own LDS
//   buffers, and at the end group 1's tiles are folded into group 0's through LDS.  The 8 waves
//   fill a CU as two 4-wave workgroups of half the split length would, with half as many
//   partials for the merge to read;
// - PG = 1, registers capped for 3 waves per SIMD (prompt sections: many chunks, where more
//   waves per SIMD cover more of each wave's dependency chain).
template <int D, int NBUF, int WPE, int PG>
__global__ __launch_bounds__(256 * PG) __attribute__((amdgpu_waves_per_eu(WPE)))
void section_i8_kernel(KVQ_PLACEMENT_PARAMS, DecodeArgs args) {
  const DecodeArgs a = KVQ_PLACED(args);
  constexpr int NW = 4;                  // waves = row tiles
  constexpr int NG = D / kGroup;         // scale groups
  constexpr int NT = D / 16;             // output tiles
  constexpr int PAGE_B = kPage * D;      // bytes of one code page
  constexpr int CH = PAGE_B / 16;        // 16-byte chunks per code page
  constexpr int CPT = 2 * CH / (NW * 64);  // chunks per thread per page (K and V together)
  constexpr int SCALE_B = kPage * NG * 2;  // bytes of one scale tile
  constexpr int SDW = SCALE_B / 4;
  static_assert(CPT >= 1 && (NBUF & 1) == 0, "page split and LDS double buffer");
  static_assert(PG == 1 || PG == 2, "page groups");
  __shared__ __attribute__((aligned(16))) h8_t s_k[PG][2][NG][64];     // K fragments [group][lane]
  __shared__ __attribute__((aligned(16))) u2_t s_v[PG][2][NT][64];     // V operands [tile][lane] (4 codes)
  __shared__ __attribute__((aligned(16))) uint32_t s_sc[PG][2][2][SDW];  // K, V scale tiles, token-quad-major
  __shared__ __attribute__((aligned(16))) float s_alpha[NW * PG][16];  // rescale factors, per row

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (NW * PG - 1);
  const int wave = wave_all & (NW - 1);  // (0 .. 3: lets the compiler fix each chunk's plane)
  const int pg = PG > 1 ? wave_all / NW : 0;  // page group: pages PG i + pg
  const int rt = wave;  // this wave's row tile
  const int n16 = lane & 15, q4 = lane >> 4;
  const int j = blockIdx.x % a.NS;
  const int h = (blockIdx.x / (a.NS * a.row_groups)) % a.Hkv;
  const int c = (blockIdx.x / (a.NS * a.row_groups * a.Hkv)) % a.chunks;
  const int s = blockIdx.x / (a.NS * a.row_groups * a.chunks * a.Hkv);
  const int c0 = c * a.qchunk;
  const int n_here = min(a.qchunk, a.nq - c0);
  const int L_full = max(0, min(context_lens[s], a.max_context_len));
  const int L = max(0, L_full - a.nq + c0 + n_here);  // the chunk attends over keys 0 .. L - 1
  const int P = (L + kPage - 1) / kPage;
  const int p0 = j * a.cpp;
  const int p1 = min(p0 + a.cpp, P);
  if (p0 >= p1) return;  // empty split (uniform): nothing written, the merge skips it
  const int n_units = p1 - p0;
  const int32_t *btrow = block_tables + (int64_t)s * a.max_blocks;
  auto page_of = [&](int k) -> int64_t {  // (pages past the split are read with size-0 resources)
    const int blk = btrow[min(p0 + k, a.max_blocks - 1)];
    return (int64_t)min(max(blk, 0), a.NB - 1) * a.Hkv + h;
  };

  // ---- this thread's share of a page: code chunks id = t + 256 ci (K if id < CH, else V; chunk
  // cc of its plane is lane cc % 64's 16 bytes at 1 KiB offset cc / 64, i.e. the decode kernel's
  // load cc / 64 of that lane), and one dword of a scale tile (wave 0: K, wave 1: V)
  u4_t cb[NBUF][CPT];
  uint32_t sb[NBUF];
  auto issue = [&](int b, int i) {
    const int k = PG * i + pg;
    const bool ok = k < n_units;  // (past the split: size-0 resources, the loads return zeros)
    const int64_t page = page_of(k);
#pragma unroll
    for (int ci = 0; ci < CPT; ++ci) {
      const int id0 = wave * 64 + NW * 64 * ci;  // the wave's first chunk (wave-uniform)
      const bool is_v = id0 >= CH;
      const auto r = page_rsrc(is_v ? a.vc : a.kc, page, PAGE_B, ok ? PAGE_B : 0);
      cb[b][ci] = ld16_page<0>(r, lane * 16, ((is_v ? id0 - CH : id0) >> 6) * 1024);
    }
    const auto rs = page_rsrc(wave == 1 ? (const void *)a.vs : (const void *)a.ks, page, SCALE_B,
                              ok && wave < 2 ? SCALE_B : 0);
    sb[b] = ld4_page<0>(rs, lane * 4, 0);
  };
  // restaged scale dword of tile dword l (group-major [group][token] -> [token quad][group][token])
  const int st_dw = (((lane & 7) >> 1) * NG + (lane >> 3)) * 2 + (lane & 1);
  auto stage = [&](int b, int lb, int i) {
    const int k = PG * i + pg;
#pragma unroll
    for (int ci = 0; ci < CPT; ++ci) {
      const int id0 = wave * 64 + NW * 64 * ci;
      const bool is_v = id0 >= CH;
      const int i = (is_v ? id0 - CH : id0) >> 6;  // the decode kernel's load index
      const u4_t w = cb[b][ci];
      if (!is_v) {
        s_k[pg][lb][2 * i][lane] = i8x8_to_h8(w[0], w[1]);
        s_k[pg][lb][2 * i + 1][lane] = i8x8_to_h8(w[2], w[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t v0, v1;
          i8x4_to_f16(w[e], v0, v1);
          s_v[pg][lb][4 * i + e][lane] = u2_t{v0, v1};  // the P.V operand as it is read
        }
      }
    }
    // V scales of tokens past the chunk's context are stored as 0: those tokens have p = 0, but
    // their codes and scales may be stale (even NaN).  Tile dword l holds tokens 2 (l % 8) and
    // 2 (l % 8) + 1 of group l / 8.
    uint32_t sw = sb[b];
    if (wave == 1) {
      const int lim = k < n_units ? min(L - (p0 + k) * kPage, kPage) : 0;
      const int t0 = 2 * (lane & 7);
      sw &= (t0 < lim ? 0xFFFFu : 0u) | (t0 + 1 < lim ? 0xFFFF0000u : 0u);
    }
    if (wave < 2 && lane < SDW) s_sc[pg][lb][wave][st_dw] = sw;
  };
  auto lds_barrier = [] {  // LDS-only fences: the page loads in flight are not waited for
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  // Q first, then the first NBUF pages
  u4_t qraw[NG];
  load_q_mq<D>(a, s, h, rt, c0, n_here, n16, q4, qraw);
#pragma unroll
  for (int b = 0; b < NBUF; ++b) {  // (in page order, and before Q is waited for)
    issue(b, b);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Q rescaled per row by 2^shift so that max |q| lies in [2^14, 2^15): exact in f16
  int shift = 0;
  {
    float qmax = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(qraw[g][e])), fabsf(bf16_hi(qraw[g][e]))));
    qmax = rows_max(qmax);
    if (qmax > 0.0f) {
      int e2;
      frexpf(qmax, &e2);
      shift = 15 - e2;
    }
  }
  h8_t qop[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qop[g][2 * e] = (_Float16)ldexpf(bf16_lo(qraw[g][e]), shift);
      qop[g][2 * e + 1] = (_Float16)ldexpf(bf16_hi(qraw[g][e]), shift);
    }
  const float cmul = ldexpf(kLog2e / sqrtf((float)D), -shift);
  // the lane's row (query token c0 + (16 rt + n16) / G) sees keys 0 .. L_row - 1
  const int L_row = L_full - a.nq + c0 + (16 * rt + n16) / a.G + 1;
  const int L_min = L_full - a.nq + c0 + 1;  // the chunk's first query token's limit (the smallest)
  // (wave-uniform) whether this wave's tile holds a real row: with fewer than 49 rows (8 query
  // tokens at G = 6) the last tile is padding, and its wave only stages pages
  const bool tile_used = 16 * rt < n_here * a.G;

  float m_run = -INFINITY, l_run = 0.0f;
  f4_t acc[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) acc[jt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto scales = [&](int lb, int which, u2_t (&out)[NG]) {
    const u4_t *src = reinterpret_cast<const u4_t *>(&s_sc[pg][lb][which][q4 * NG * 2]);
#pragma unroll
    for (int i = 0; i < NG / 2; ++i) {
      const u4_t w = src[i];
      out[2 * i] = u2_t{w[0], w[1]};
      out[2 * i + 1] = u2_t{w[2], w[3]};
    }
  };

  // One page from LDS buffer lb: Q.K^T, one online-softmax update, P.V (the decode kernel's step).
  auto process = [&](int lb, int i) {
    const int k = PG * i + pg;
    // valid tokens of the page for this lane's row
    const int lim_row = k < n_units ? min(max(L_row - (p0 + k) * kPage, 0), kPage) : 0;
    u2_t ksc[NG];
    scales(lb, 0, ksc);
    f4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto scale_group = [&](int g, const f4_t &cg) {
      const u2_t sw = ksc[g];
      sc[0] = fma_h16lo(sw[0], cg[0], sc[0]);
      sc[1] = fma_h16hi(sw[0], cg[1], sc[1]);
      sc[2] = fma_h16lo(sw[1], cg[2], sc[2]);
      sc[3] = fma_h16hi(sw[1], cg[3], sc[3]);
      pin4(sc);
    };
    f4_t c_prev = mfma_f16(s_k[pg][lb][0][lane], qop[0], f4_t{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
    for (int g = 1; g < NG; ++g) {
      const f4_t cg = mfma_f16(s_k[pg][lb][g][lane], qop[g], f4_t{0.0f, 0.0f, 0.0f, 0.0f});
      scale_group(g - 1, c_prev);
      c_prev = cg;
    }
    scale_group(NG - 1, c_prev);
    float x[4];
    if (k < n_units && (p0 + k + 1) * kPage <= L_min) {  // (uniform) every row sees the whole page
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = sc[i] * cmul;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (4 * q4 + i < lim_row) ? sc[i] * cmul : -INFINITY;
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = rows_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = (m_new == m_run) ? 1.0f : exp2_w(m_run - m_use);
    const bool grew = alpha != 1.0f && m_run != -INFINITY;
    float p[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2_w(x[i] - m_use);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(grew)) {  // some row's maximum grew: rescale its accumulator rows
      if (q4 == 0) s_alpha[wave_all][n16] = alpha;
      const f4_t ar = *reinterpret_cast<const f4_t *>(&s_alpha[wave_all][4 * q4]);
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) acc[jt] *= ar;
    }
    // P.V: P' = p * s_v per (token, group) as f16 hi + lo times the exact f16 V codes (the V
    // scales of tokens past the chunk's context were staged as 0)
    u2_t vsc[NG];
    scales(lb, 1, vsc);
    const h2_t ph01 = {(_Float16)p[0], (_Float16)p[1]}, ph23 = {(_Float16)p[2], (_Float16)p[3]};
    const h2_t pl01 = {(_Float16)(p[0] - (float)ph01[0]), (_Float16)(p[1] - (float)ph01[1])};
    const h2_t pl23 = {(_Float16)(p[2] - (float)ph23[0]), (_Float16)(p[3] - (float)ph23[1])};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const u2_t sv = vsc[g];
      const uint32_t w01 = sv[0], w23 = sv[1];
      const h2_t s01 = __builtin_bit_cast(h2_t, w01), s23 = __builtin_bit_cast(h2_t, w23);
      const h2_t hi01 = ph01 * s01, hi23 = ph23 * s23;
      const h2_t lo01 = __builtin_elementwise_fma(pl01, s01, __builtin_elementwise_fma(ph01, s01, -hi01));
      const h2_t lo23 = __builtin_elementwise_fma(pl23, s23, __builtin_elementwise_fma(ph23, s23, -hi23));
      // two K = 16 products on one read of the V operand (hi, then lo): the 8-byte operand is
      // read from LDS once, where the K = 32 form packing hi and lo needs the codes twice
      const h4_t ph = __builtin_bit_cast(h4_t, u2_t{__builtin_bit_cast(uint32_t, hi01), __builtin_bit_cast(uint32_t, hi23)});
      const h4_t pl = __builtin_bit_cast(h4_t, u2_t{__builtin_bit_cast(uint32_t, lo01), __builtin_bit_cast(uint32_t, lo23)});
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int jt = 2 * g + jj;
        const h4_t vb = __builtin_bit_cast(h4_t, s_v[pg][lb][jt][lane]);
        acc[jt] = mfma16_f16(ph, vb, acc[jt]);
        acc[jt] = mfma16_f16(pl, vb, acc[jt]);
      }
    }
  };

  // Step k: one barrier (page k is in LDS buffer k % 2, and every wave is done with page k - 1),
  // then every wave's step on its tile for page k together with the staging of page k + 1 (its
  // registers, buffer (k + 1) % NBUF, into LDS buffer (k + 1) % 2, which held page k - 1), so
  // that the conversion overlaps the matrix products; the register buffer is then refilled with
  // page k + 1 + NBUF.  The trip count is the same for every wave and a multiple of NBUF with no
  // early exit: pages past the split's end read zeros and are fully masked (p = 0), which keeps
  // the buffers in fixed registers and the waits for each page exact.
  stage(0, 0, 0);
  issue(0, NBUF);
  const int n_steps = (n_units + PG - 1) / PG;  // pages per group (the same trip count for every wave)
  for (int i0 = 0; i0 < n_steps; i0 += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int i = i0 + b;
      lds_barrier();
      if (tile_used) process(b & 1, i);  // (a tile of padding rows only stages)
      stage((b + 1) % NBUF, (b + 1) & 1, i + 1);
      issue((b + 1) % NBUF, i + 1 + NBUF);
    }
  }
  if constexpr (PG > 1) {
    // Two page groups: group 1's tiles (accumulators over the staging buffers, and (m, l) per row)
    // are folded into group 0's, each weighted by 2^(m - M) per row with M the larger maximum; group
    // 0 then stores the tile's partial as one group would.
    __shared__ float s_xm[2][NW][16], s_xl[NW][16];
    lds_barrier();  // every wave is done with the staging buffers
    const float l_row = rows_sum(l_run);
    if (q4 == 0) {
      s_xm[pg][rt][n16] = m_run;
      if (pg == 1) s_xl[rt][n16] = l_row;
    }
    f4_t *xk = reinterpret_cast<f4_t *>(&s_k[0][0][0][0]);  // tiles 0 .. NT / 2 - 1
    f4_t *xv = reinterpret_cast<f4_t *>(&s_v[0][0][0][0]);  // tiles NT / 2 .. NT - 1
    if (pg == 1 && tile_used) {
#pragma unroll
      for (int jt = 0; jt < NT / 2; ++jt) xk[(rt * (NT / 2) + jt) * 64 + lane] = acc[jt];
#pragma unroll
      for (int jt = NT / 2; jt < NT; ++jt) xv[(rt * (NT / 2) + jt - NT / 2) * 64 + lane] = acc[jt];
    }
    lds_barrier();
    if (pg == 1 || !tile_used) return;
    const f4_t m0r = *reinterpret_cast<const f4_t *>(&s_xm[0][rt][4 * q4]);
    const f4_t m1r = *reinterpret_cast<const f4_t *>(&s_xm[1][rt][4 * q4]);
    f4_t w0, w1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float M = fmaxf(m0r[r], m1r[r]);
      w0[r] = (m0r[r] == -INFINITY) ? 0.0f : exp2_w(m0r[r] - M);  // (a group without keys: 0)
      w1[r] = (m1r[r] == -INFINITY) ? 0.0f : exp2_w(m1r[r] - M);
    }
#pragma unroll
    for (int jt = 0; jt < NT / 2; ++jt) acc[jt] = acc[jt] * w0 + xk[(rt * (NT / 2) + jt) * 64 + lane] * w1;
#pragma unroll
    for (int jt = NT / 2; jt < NT; ++jt) acc[jt] = acc[jt] * w0 + xv[(rt * (NT / 2) + jt - NT / 2) * 64 + lane] * w1;
    const float m1 = s_xm[1][rt][n16], l1 = s_xl[rt][n16];
    const float Mn = fmaxf(m_run, m1);
    const float a0 = (m_run == -INFINITY) ? 0.0f : exp2_w(m_run - Mn);
    const float a1 = (m1 == -INFINITY) ? 0.0f : exp2_w(m1 - Mn);
    m_run = Mn;
    l_run = (q4 == 0) ? fmaf(a0, l_row, a1 * l1) : 0.0f;  // (summed over the row's lanes when stored)
  }
  // The epilogue takes its lane indices from a fresh lane count (behind an opaque mask, so that it
  // is not merged with the prologue's): keeping the prologue's lane-derived values live across the
  // page loop would push them out of the capped register budget.
  unsigned all = ~0u;
  asm volatile("" : "+s"(all));
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(all, __builtin_amdgcn_mbcnt_lo(all, 0u));
  write_partial<D, NW, true, NW>(a, s, h, j, wave, lane_e & 15, lane_e >> 4, m_run, l_run, acc, nullptr, rt, c0,
                                 n_here);
}

// ---- BF16 cache: 1-page units, bf16 MFMA (Q.K exact; P as bf16 hi + lo)
__device__ __forceinline__ f4_t mfma16_bf16(s4_t a, s4_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_bf16_kernel(KVQ_PLACEMENT_PARAMS, DecodeArgs args) {
  const DecodeArgs a = KVQ_PLACED(args);
  constexpr int NG = D / 32;  // 16-byte loads per lane per page (8 bf16 each)
  constexpr int NT = D / 16;
  constexpr int PAGE_B = kPage * D * 2;
  __shared__ __attribute__((aligned(16))) float s_alpha[NW][16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, q4 = lane >> 4;
  const int j = blockIdx.x % a.NS;
  const int h = (blockIdx.x / a.NS) % a.Hkv;
  const int s = blockIdx.x / (a.NS * a.Hkv);
  const int p0 = j * a.cpp;
  const int32_t *btrow = block_tables + (int64_t)s * a.max_blocks;
  // the block id of the wave's first page, Q and the new token's rows are requested together with
  // the context length (the id's index is clamped to the table row, not to the context)
  const int blk0 = btrow[min(p0 + wave, a.max_blocks - 1)];
  u4_t qraw[NG];
  load_q<D>(a, s, h, n16, q4, qraw);
  u2_t knew, vnew;
  load_new_rows<D>(a, s, h, a.k_new != nullptr, lane, knew, vnew);
  const int L = max(0, min(context_lens[s], a.max_context_len));
  const int P = (L + kPage - 1) / kPage;
  const int p1 = min(p0 + a.cpp, P);
  if (p0 >= p1) return;  // empty split: nothing written, the merge skips it
  const int n_units = p1 - p0;
  const bool head_ok = n16 < a.G;

  // The wave that holds the sequence's last page writes the step's new token into it before it
  // requests that page (unit k_last of the wave).
  const int blk_last = btrow[P - 1];
  // (a length above max_context_len, outside the contract, writes nothing)
  const bool own_new = a.k_new != nullptr && context_lens[s] <= a.max_context_len && p1 == P &&
                       wave == (n_units - 1) % NW && blk_last >= 0 && blk_last < a.NB;
  const int k_last = (n_units - 1) / NW;
  const int64_t page_new = (int64_t)blk_last * a.Hkv + h;
  const int t_new = (L - 1) & (kPage - 1);
  b8_t qop[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) qop[g] = __builtin_bit_cast(b8_t, qraw[g]);
  const float cmul = kLog2e / sqrtf((float)D);

  float m_run = -INFINITY, l_run = 0.0f;
  f4_t acc[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) acc[jt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int voff = lane * 16;
  auto page_index_of = [&](int blk) -> int64_t { return (int64_t)min(max(blk, 0), a.NB - 1) * a.Hkv + h; };
  auto page_index = [&](int p) -> int64_t { return page_index_of(btrow[min(p, a.max_blocks - 1)]); };
  u4_t kb[NG], vb[NG];
  auto load = [&](u4_t(&dst)[NG], const void *base, int64_t pg, bool ok) {
    const auto r = page_rsrc(base, pg, PAGE_B, ok ? PAGE_B : 0);
#pragma unroll
    for (int i = 0; i < NG; ++i) dst[i] = ld16_page<kStreamPolicy>(r, voff, 1024 * i);
  };
  int u = wave;
  // The owner's stores complete (vmcnt, in issue order) before it requests the page they go to:
  // here when that page is its first, else before that page's K load below.
  if (own_new && k_last == 0) {
    write_new_bf16<D>(a, page_new, t_new, knew, vnew, lane);
    wait_vmcnt<0>();
  }
  {
    const bool ok = u < n_units;
    const int64_t pg = page_index_of(blk0);
    load(kb, a.kc, pg, ok);
    load(vb, a.vc, pg, ok);
  }
  if (own_new && k_last != 0) write_new_bf16<D>(a, page_new, t_new, knew, vnew, lane);
  for (; u < n_units; u += NW) {
    const int lim = min(L - (p0 + u) * kPage, kPage);
    const int un = u + NW;
    const bool next_ok = un < n_units;
    const int64_t pgn = page_index(p0 + un);

    f4_t score = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < NG; ++g) score = mfma_bf16(__builtin_bit_cast(b8_t, kb[g]), qop[g], score);
    if (own_new && un == n_units - 1) {
      // outstanding now: this page's V loads, issued after the stores unless this is the wave's
      // first page (then the stores came after them)
      if (k_last == 1) wait_vmcnt<0>();
      else wait_vmcnt<NG>();
    }
    load(kb, a.kc, pgn, next_ok);

    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (head_ok && 4 * q4 + i < lim) ? score[i] * cmul : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = rows_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = (m_new == m_run) ? 1.0f : exp2_w(m_run - m_use);
    float p[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2_w(x[i] - m_use);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
      if (q4 == 0) s_alpha[wave][n16] = alpha;
      const f4_t ar = *reinterpret_cast<const f4_t *>(&s_alpha[wave][4 * q4]);
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) acc[jt] *= ar;
    }
    s4_t phi, plo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 hi = (__bf16)p[i];
      phi[i] = __builtin_bit_cast(short, hi);
      plo[i] = __builtin_bit_cast(short, (__bf16)(p[i] - (float)hi));
    }
    // tokens at or past lim may hold any bits (NaN): zero them in the V operand
    const uint32_t keep_lo = (4 * q4 + 0 < lim ? 0x0000FFFFu : 0u) | (4 * q4 + 1 < lim ? 0xFFFF0000u : 0u);
    const uint32_t keep_hi = (4 * q4 + 2 < lim ? 0x0000FFFFu : 0u) | (4 * q4 + 3 < lim ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      const uint32_t w0 = vb[jt >> 1][(jt & 1) * 2] & keep_lo;
      const uint32_t w1 = vb[jt >> 1][(jt & 1) * 2 + 1] & keep_hi;
      const s4_t bv = __builtin_bit_cast(s4_t, u2_t{w0, w1});
      acc[jt] = mfma16_bf16(phi, bv, acc[jt]);
      acc[jt] = mfma16_bf16(plo, bv, acc[jt]);
    }
    load(vb, a.vc, pgn, next_ok);
  }
  extern __shared__ float s_merge[];  // [NW][G*D + 32] floats (dynamic)
  write_partial<D, NW>(a, s, h, j, wave, n16, q4, m_run, l_run, acc, s_merge);
}

// ------------------------------------------------------------------ decode: merge
//
// One wavefront per (64-channel chunk, output row, sequence); an output row is a (query token,
// query head) pair (one query token per sequence unless nq > 1).  The splits are taken MB at a
// time (MB = 8, 16, 32 or 64: the smallest that holds all splits, so few splits cost few loads):
// lane j loads split j's (m, l) and every lane loads its channel of all MB partial outputs, all in
// one round trip.  The block's maximum and weights w_j = 2^(m_j - M) come from wave reductions,
// each lane folds the MB partials with the weights broadcast from their lanes, and blocks beyond
// the first (more than 64 splits) are folded with the online softmax's rescaling.  Only the
// splits that hold pages count (their number follows from the row's context length, read
// alongside the partials):  out = o / l;  lse = ln 2 * (M + log2 l).

// Reductions over a wavefront: DPP within each 16-lane row (pairs, quads, half rows, rows), then
// the four row results read into scalars.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_lane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  return fmaxf(fmaxf(row_lane(x, 0), row_lane(x, 16)), fmaxf(row_lane(x, 32), row_lane(x, 48)));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return (row_lane(x, 0) + row_lane(x, 16)) + (row_lane(x, 32) + row_lane(x, 48));
}

template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

template <int D, int MB>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float *__restrict__ o_part,
                                                           const float2 *__restrict__ mlp,
                                                           const int32_t *__restrict__ cl, int Hq, int nq, int NS,
                                                           DecodeArgs a) {
  constexpr int NCH = D / 64;
  // What the partials' requests need leads the argument list (the hardware preloads it into scalar
  // registers at launch).  The other arguments are read at the top in one batch: passed through an
  // empty asm (tied operands, no side effects), they are all loaded before it.  Left alone, the
  // compiler reads each one where it is first needed and waits there, which adds a round trip.
  float *outp = a.out, *lsep = a.lse;
  int qchunk = a.qchunk, mcl = a.max_context_len, cpp = a.cpp;
  asm("; merge arguments" : "+s"(outp), "+s"(lsep), "+s"(qchunk), "+s"(mcl), "+s"(cpp));
  // (the compiler takes asm results as varying across lanes; they are not)
  outp = uniform_ptr(outp);
  lsep = uniform_ptr(lsep);
  qchunk = __builtin_amdgcn_readfirstlane(qchunk);
  mcl = __builtin_amdgcn_readfirstlane(mcl);
  cpp = __builtin_amdgcn_readfirstlane(cpp);
  const int lane = threadIdx.x;
  const int HQ = Hq * nq;  // output rows per sequence: (query token, query head)
  const int chunk = blockIdx.x % NCH;
  const int hq = (blockIdx.x / NCH) % HQ;
  const int s = blockIdx.x / (NCH * HQ);
  const int c = chunk * 64 + lane;
  const int64_t orow = ((int64_t)s * HQ + hq);
  const int64_t base = orow * NS;
  // buffer loads over this row's partials (past NS they return 0 and are masked below)
  const auto rml = __builtin_amdgcn_make_buffer_rsrc(const_cast<float2 *>(mlp + base), 0, NS * 8, 0x00020000);
  const auto ro = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(o_part + base * D), 0, NS * D * 4, 0x00020000);
  // the row's query chunk attends over the keys up to its last query token: the context length
  // that sets the row's splits
  const int Lc = cl[s];
  const int qi = hq / Hq;  // query token of the row
  const int c0 = qi - qi % qchunk, n_here = min(qchunk, nq - c0);
  float M = -INFINITY, l = 0.0f, o = 0.0f;
  static_assert(MB >= 8 && MB <= 64 && (MB & (MB - 1)) == 0, "split block: 8, 16, 32 or 64");
  for (int j0 = 0; j0 < NS; j0 += MB) {
    const u2_t w = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(rml, lane * 8, j0 * 8, 0));
    float ov[MB];
#pragma unroll
    for (int u = 0; u < MB; ++u)
      ov[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, c * 4, (j0 + u) * D * 4, 0));
    // (read here, after the partial loads are issued: the wait for the context length then does
    // not hold them back)
    const int Lk = __builtin_amdgcn_readfirstlane(Lc);
    const int L = max(0, min(max(0, min(Lk, mcl)) - nq + c0 + n_here, mcl));
    const int nsa = min(NS, ((L + kPage - 1) / kPage + cpp - 1) / cpp);  // splits with pages
    // splits past nsa were not written by this call: their (m, l, o) are masked, never multiplied
    const int nb = nsa - j0;
    const bool valid = lane < nb && lane < MB;  // (lanes past the block read the next one's)
    const float mj = valid ? __uint_as_float(w[0]) : -INFINITY;
    const float Mn = fmaxf(M, wave_max(mj));
    const float Mr = (Mn == -INFINITY) ? 0.0f : Mn;  // (no key yet: any finite reference)
    const float alpha = exp2_w(M - Mr);                // M = -inf: 0
    const float wj = exp2_w(mj - Mr);                  // mj = -inf: 0
    l = fmaf(l, alpha, wave_sum(valid ? wj * __uint_as_float(w[1]) : 0.0f));
    float acc = o * alpha;
    if (nb >= MB) {
#pragma unroll
      for (int u = 0; u < MB; ++u) acc = fmaf(row_lane(wj, u), ov[u], acc);
    } else {
#pragma unroll
      for (int u = 0; u < MB; ++u) acc = fmaf(row_lane(wj, u), (u < nb) ? ov[u] : 0.0f, acc);
    }
    o = acc;
    M = Mn;
  }
  if (M == -INFINITY) {  // no split holds a key: empty context
    outp[orow * D + c] = 0.0f;
    if (lsep && chunk == 0 && lane == 0) lsep[orow] = -INFINITY;
  } else {
    outp[orow * D + c] = o / l;
    if (lsep && chunk == 0 && lane == 0) lsep[orow] = kLn2 * (M + log2f(l));
  }
}

// ------------------------------------------------------------------ fixed scratch
//
// Device scratch of kvq_decode_step_noalloc (for callers that cannot allocate): the split
// partials live in this file-scope array instead of a caller's workspace.  Each device that loads
// the library holds its own copy, zero-initialised when the code object is loaded, until the
// process ends.  Host code must never pass the array's name to a kernel (on the host it names a
// stand-in, not device memory): scratch_address() returns the device address of the current
// device's copy, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void **ptr) {
  constexpr int kMaxDevices = 64;
  static void *addr[kMaxDevices] = {};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------------ launchers

// A writer with its leading arguments ahead of the argument block.
template <typename Kernel>
static void launch_write(Kernel kernel, dim3 grid, dim3 block, hipStream_t stream, const WriteArgs &a) {
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, a.k, a.v, a.slot_mapping, a.T, a.Hkv, a);
}

hipError_t launch_kv_write(int dtype, const WriteArgs &a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (dtype == 2 && a.T < kPage) {  // per-head INT8, few tokens: one wavefront per row, 4 rows per block
    const unsigned grid = (unsigned)(((int64_t)a.T * a.Hkv * 2 + 3) / 4);
    if (a.D == 256) launch_write(kv_write_i8h_kernel<256>, dim3(grid), dim3(256), stream, a);
    else launch_write(kv_write_i8h_kernel<128>, dim3(grid), dim3(256), stream, a);
    return hipGetLastError();
  }
  if (dtype == 2) {
    const dim3 grid((unsigned)((a.T + kPage - 1) / kPage), (unsigned)a.Hkv);
    if (a.D == 256) launch_write((kv_write_i8_kernel<256, 1>), grid, dim3(256), stream, a);
    else launch_write((kv_write_i8_kernel<128, 1>), grid, dim3(128), stream, a);
    return hipGetLastError();
  }
  if (a.T < kPage) {  // no whole page possible: the per-group writers have the shortest latency
    const int per = (dtype == 0 ? a.D / kGroup : a.D / 8) * 2;
    const unsigned grid = (unsigned)(((int64_t)a.T * a.Hkv * per + 255) / 256);
    if (dtype == 0) {
      if (a.D == 256) launch_write(kv_write_i8_rows_kernel<256>, dim3(grid), dim3(256), stream, a);
      else launch_write(kv_write_i8_rows_kernel<128>, dim3(grid), dim3(256), stream, a);
    } else {
      if (a.D == 256) launch_write(kv_write_bf16_rows_kernel<256>, dim3(grid), dim3(256), stream, a);
      else launch_write(kv_write_bf16_rows_kernel<128>, dim3(grid), dim3(256), stream, a);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.T + kPage - 1) / kPage), (unsigned)a.Hkv);
  if (dtype == 0) {
    if (a.D == 256) launch_write((kv_write_i8_kernel<256, 0>), grid, dim3(256), stream, a);
    else launch_write((kv_write_i8_kernel<128, 0>), grid, dim3(128), stream, a);
  } else {
    if (a.D == 256) launch_write(kv_write_bf16_kernel<256>, grid, dim3(256), stream, a);
    else launch_write(kv_write_bf16_kernel<128>, grid, dim3(128), stream, a);
  }
  return hipGetLastError();
}

// A decode split kernel with its placement arguments ahead of the argument block.
template <typename Kernel>
static void launch_placed(Kernel kernel, unsigned grid, unsigned block, size_t smem, hipStream_t stream,
                          const DecodeArgs &a) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), smem, stream, a.block_tables, a.context_lens, a.NS, a.Hkv,
                     a.cpp, a.max_blocks, a.row_groups, a.chunks, a.qchunk, a.nq, a);
}

template <int D, int NW, bool I8, int FMT = 0>
static void launch_split(const DecodeArgs &a, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.S * a.Hkv * a.NS);
  const size_t smem = NW > 1 ? (size_t)NW * merge_stride<D>() * sizeof(float) : 0;  // merge scratch
  if constexpr (I8)
    launch_placed(decode_split_i8_kernel<D, NW, 0, FMT>, grid, NW * 64, smem, stream, a);
  else
    launch_placed(decode_split_bf16_kernel<D, NW>, grid, NW * 64, smem, stream, a);
}

template <int D, bool I8>
static void launch_split_nw(const DecodeArgs &a, hipStream_t stream) {
  switch (a.waves) {
    case 1: launch_split<D, 1, I8>(a, stream); break;
    case 2: launch_split<D, 2, I8>(a, stream); break;
    case 8: launch_split<D, 8, I8>(a, stream); break;
    default: launch_split<D, 4, I8>(a, stream); break;
  }
}

// Several query tokens per sequence (INT8 cache): one workgroup per (group of rtw 16-row tiles,
// split, KV head, query chunk, sequence).
template <int D, int FMT>
static void launch_split_mq(const DecodeArgs &a, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.S * a.chunks * a.Hkv * a.row_groups * a.NS);
  const size_t smem = (size_t)4 * merge_stride<D>() * sizeof(float);  // LDS merge of 4 waves' tiles
  if (a.rtw == 4 && FMT == 0 && a.chunks > 1)  // q8_0 prompt sections: 3 waves per SIMD
    launch_placed(section_i8_kernel<D, 2, 3, 1>, grid, 256, 0, stream, a);
  else if (a.rtw == 4 && FMT == 0)  // q8_0 single chunk: two page groups of 4 waves
    launch_placed(section_i8_kernel<D, 2, 2, 2>, grid, 512, 0, stream, a);
  else if (a.rtw == 4)  // (one wave per tile: no merge scratch, so several workgroups share a CU)
    launch_placed(decode_split_i8_kernel<D, 4, 4, FMT>, grid, 256, 0, stream, a);
  else if (a.rtw == 2)  // (8 waves, 4 per tile: twice the waves per SIMD at the same split count)
    launch_placed(decode_split_i8_kernel<D, 8, 2, FMT>, grid, 512, 2 * smem, stream, a);
  else
    launch_placed(decode_split_i8_kernel<D, 4, 1, FMT>, grid, 256, smem, stream, a);
}

// dtype: 0 INT8 q8_0, 1 BF16, 2 INT8 per-head
hipError_t launch_decode_split(int dtype, const DecodeArgs &a, hipStream_t stream) {
  if (dtype == 0 && a.nq > 1) {
    if (a.D == 256) launch_split_mq<256, 0>(a, stream);
    else launch_split_mq<128, 0>(a, stream);
  } else if (dtype == 2 && a.nq > 1) {
    if (a.D == 256) launch_split_mq<256, 1>(a, stream);
    else launch_split_mq<128, 1>(a, stream);
  } else if (dtype == 2) {
    if (a.D == 256) launch_split<256, 4, true, 1>(a, stream);
    else launch_split<128, 4, true, 1>(a, stream);
  } else if (dtype == 0 && a.int_qk) {
    if (a.D == 256) launch_split<256, 4, true, 2>(a, stream);
    else launch_split<128, 4, true, 2>(a, stream);
  } else if (dtype == 0) {
    if (a.D == 256) launch_split_nw<256, true>(a, stream);
    else launch_split_nw<128, true>(a, stream);
  } else {
    if (a.D == 256) launch_split_nw<256, false>(a, stream);
    else launch_split_nw<128, false>(a, stream);
  }
  return hipGetLastError();
}

template <int D, int MB>
static void launch_merge(const DecodeArgs &a, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_merge_kernel<D, MB>), dim3(grid), dim3(64), 0, stream, a.o_part, a.ml, a.context_lens,
                     a.Hq, a.nq, a.NS, a);
}

template <int D>
static void launch_merge_mb(const DecodeArgs &a, unsigned grid, hipStream_t stream) {
  if (a.NS <= 8) launch_merge<D, 8>(a, grid, stream);
  else if (a.NS <= 16) launch_merge<D, 16>(a, grid, stream);
  else if (a.NS <= 32) launch_merge<D, 32>(a, grid, stream);
  else launch_merge<D, 64>(a, grid, stream);
}

hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.S * a.Hq * a.nq * (a.D / 64));
  if (a.D == 256) launch_merge_mb<256>(a, grid, stream);
  else launch_merge_mb<128>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace kvq
