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

#include "kvq_internal.h"
#include "kvq_layout.h"

namespace kvq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Four int8 codes (one dword) -> four exact f16 values, as two f16x2 words.
// (x ^ 0x80) is x + 128 as an unsigned byte; 0x6400 | u is the f16 1024 + u; subtracting
// 1152 gives x exactly.
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, uint32_t &lo, uint32_t &hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = (u & 0x000000FFu) | ((u & 0x0000FF00u) << 8) | 0x64006400u;
  const uint32_t b = ((u & 0x00FF0000u) >> 16) | ((u & 0xFF000000u) >> 8) | 0x64006400u;
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

__device__ __forceinline__ f4_t mfma_bf16(b8_t a, b8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp16 number e of a lane's scale block (packed in 16-byte words).
template <int N>
__device__ __forceinline__ float scale_at(const u4_t (&w)[N], int e) {
  const uint32_t d = w[e >> 3][(e >> 1) & 3];
  return f16_bits_to_f32((e & 1) ? (d >> 16) : (d & 0xFFFFu));
}

// ------------------------------------------------------------------ quantize-on-write

// One thread per (token, KV head, K or V, 32-channel group).
template <int D>
__global__ __launch_bounds__(256) void kv_write_i8_kernel(WriteArgs a) {
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
  const float d = fminf(amax / 127.0f, 65504.0f);
  const _Float16 s16 = (_Float16)d;
  const float s = (float)s16;
  uint32_t packed[kGroup / 4];
#pragma unroll
  for (int i = 0; i < kGroup / 4; ++i) packed[i] = 0u;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    float q = 0.0f;
    if (s != 0.0f) {
      q = __builtin_rintf(x[i] / s);
      if (q != q) q = 0.0f;
      q = fminf(fmaxf(q, -127.0f), 127.0f);
    }
    packed[i >> 2] |= ((uint32_t)(int)q & 0xFFu) << (8 * (i & 3));
  }
  const int64_t page = (int64_t)blk * a.Hkv + h;
  const uint16_t sbits = __builtin_bit_cast(uint16_t, s16);
  if (which == 0) {
    int8_t *dst = static_cast<int8_t *>(a.kc) + page * (kPage * D);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      u2_t w = {packed[2 * qq], packed[2 * qq + 1]};
      *reinterpret_cast<u2_t *>(dst + i8_k_offset(off, kGroup * g + 8 * qq)) = w;
    }
    a.ks[(page * kPage + off) * NG + g] = sbits;
  } else {
    int8_t *dst = static_cast<int8_t *>(a.vc) + page * (kPage * D);
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
      dst[i8_v_offset(off, kGroup * g + i)] = (int8_t)((packed[i >> 2] >> (8 * (i & 3))) & 0xFFu);
    a.vs[(page * kPage + off) * NG + g] = sbits;
  }
}

// BF16 cache: one thread per (token, KV head, K or V, 8-channel chunk); a scatter copy.
template <int D>
__global__ __launch_bounds__(256) void kv_write_bf16_kernel(WriteArgs a) {
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

// ------------------------------------------------------------------ decode: split partials
//
// Workgroup (split j, KV head h, sequence s) of NW wavefronts.  The split owns pages
// [j*cpp, min((j+1)*cpp, ceil(L/16))); the waves take 2-page units round-robin.  Within a
// wavefront, lane l = 16*q4 + n16:
//   Q.K   (A = K codes, B = Q):   lane holds scores of head n16, tokens 4*q4 .. 4*q4+3
//   P.V   (A = P',      B = V):   A lane holds P' of head n16 for K-slots (page pg, token
//                                 4*q4 + i) at element 4*pg + i -- the Q.K result layout
//   acc   (P.V result):           lane holds heads 4*q4 .. 4*q4+3 of channel 16*jt + n16
// Each split writes an unnormalised partial o = sum_t 2^(x_t - m) v_t with m = max_t x_t,
// x_t = log2(e) * q.k_t / sqrt(D), and l = sum_t 2^(x_t - m).
template <int D, int NW, bool I8>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(DecodeArgs a) {
  constexpr int NG = D / kGroup;  // 32-channel groups / MFMA K-chunks
  constexpr int NT = D / 16;      // 16-channel output tiles
  constexpr int NL = I8 ? D / 64 : D / 32;  // 16-byte loads per lane per page
  constexpr int NSW = NG / 2;     // 16-byte words of one lane's page scales (4 tokens x NG fp16)

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int bid = blockIdx.x;
  const int j = bid % a.NS;
  const int h = (bid / a.NS) % a.Hkv;
  const int s = bid / (a.NS * a.Hkv);
  int L = a.context_lens[s];
  L = max(0, min(L, a.max_context_len));
  const int P = (L + kPage - 1) / kPage;
  const int p0 = j * a.cpp;
  const int p1 = min(p0 + a.cpp, P);
  if (p0 >= p1) return;  // empty split: nothing written, the merge skips it
  const int n_units = (p1 - p0 + 1) >> 1;
  const int G = a.G;
  const bool head_ok = n16 < G;
  const int hq = h * G + (head_ok ? n16 : 0);

  // ---- Q operand (B of Q.K): lane holds head n16, channels 32g + 8*q4 + 0..7 of chunk g
  const uint16_t *qrow = a.q + ((int64_t)s * a.Hq + hq) * D;
  u4_t qraw[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    qraw[g] = head_ok ? *reinterpret_cast<const u4_t *>(qrow + kGroup * g + 8 * q4) : u4_t{0u, 0u, 0u, 0u};
  }
  h8_t qop[I8 ? NG : 1];
  b8_t qopb[I8 ? 1 : NG];
  float cmul;
  if constexpr (I8) {
    float qmax = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(qraw[g][e])), fabsf(bf16_hi(qraw[g][e]))));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 16));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
    int shift = 0;
    if (qmax > 0.0f) {
      int e2;
      frexpf(qmax, &e2);
      shift = 15 - e2;  // max |q| * 2^shift lies in [2^14, 2^15): exact in f16
    }
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qop[g][2 * e] = (_Float16)ldexpf(bf16_lo(qraw[g][e]), shift);
        qop[g][2 * e + 1] = (_Float16)ldexpf(bf16_hi(qraw[g][e]), shift);
      }
    cmul = head_ok ? ldexpf(kLog2e / sqrtf((float)D), -shift) : 0.0f;
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g) qopb[g] = __builtin_bit_cast(b8_t, qraw[g]);
    cmul = head_ok ? kLog2e / sqrtf((float)D) : 0.0f;
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f4_t acc[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) acc[jt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int32_t *btrow = a.block_tables + (int64_t)s * a.max_blocks;
  constexpr int kPageBytes = kPage * D * (I8 ? 1 : 2);

  for (int u = wave; u < n_units; u += NW) {
    const int pa = p0 + 2 * u;
    const bool b_ok = pa + 1 < p1;
    int ba = btrow[pa];
    int bb = b_ok ? btrow[pa + 1] : ba;
    ba = min(max(ba, 0), a.NB - 1);
    bb = min(max(bb, 0), a.NB - 1);
    const int64_t pga = (int64_t)ba * a.Hkv + h, pgb = (int64_t)bb * a.Hkv + h;

    // ---- loads: codes with one 16-byte load per lane per instruction (1 KiB per wave)
    const u4_t *KA = reinterpret_cast<const u4_t *>(static_cast<const char *>(a.kc) + pga * kPageBytes) + lane;
    const u4_t *KB = reinterpret_cast<const u4_t *>(static_cast<const char *>(a.kc) + pgb * kPageBytes) + lane;
    const u4_t *VA = reinterpret_cast<const u4_t *>(static_cast<const char *>(a.vc) + pga * kPageBytes) + lane;
    const u4_t *VB = reinterpret_cast<const u4_t *>(static_cast<const char *>(a.vc) + pgb * kPageBytes) + lane;
    u4_t kA[NL], kB[NL], vA[NL], vB[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      kA[i] = KA[64 * i];
      kB[i] = KB[64 * i];
    }
    u4_t ksA[I8 ? NSW : 1], ksB[I8 ? NSW : 1], vsA[I8 ? NSW : 1], vsB[I8 ? NSW : 1];
    if constexpr (I8) {
      const u4_t *SA = reinterpret_cast<const u4_t *>(a.ks + pga * (kPage * NG) + 4 * q4 * NG);
      const u4_t *SB = reinterpret_cast<const u4_t *>(a.ks + pgb * (kPage * NG) + 4 * q4 * NG);
#pragma unroll
      for (int i = 0; i < NSW; ++i) {
        ksA[i] = SA[i];
        ksB[i] = SB[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      vA[i] = VA[64 * i];
      vB[i] = VB[64 * i];
    }
    if constexpr (I8) {
      const u4_t *SA = reinterpret_cast<const u4_t *>(a.vs + pga * (kPage * NG) + 4 * q4 * NG);
      const u4_t *SB = reinterpret_cast<const u4_t *>(a.vs + pgb * (kPage * NG) + 4 * q4 * NG);
#pragma unroll
      for (int i = 0; i < NSW; ++i) {
        vsA[i] = SA[i];
        vsB[i] = SB[i];
      }
    }

    // ---- Q.K^T: scores of head n16 for tokens 4*q4 + i of both pages
    f4_t sc[2];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const u4_t(&kr)[NL] = pg ? kB : kA;
      f4_t score = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (I8) {
        const u4_t(&sr)[NSW] = pg ? ksB : ksA;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const h8_t av = i8x8_to_h8(kr[g >> 1][(g & 1) * 2], kr[g >> 1][(g & 1) * 2 + 1]);
          const f4_t c = mfma_f16(av, qop[g], f4_t{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
          for (int i = 0; i < 4; ++i) score[i] = fmaf(scale_at(sr, i * NG + g), c[i], score[i]);
        }
      } else {
#pragma unroll
        for (int g = 0; g < NG; ++g) score = mfma_bf16(__builtin_bit_cast(b8_t, kr[g]), qopb[g], score);
      }
      sc[pg] = score;
    }

    // ---- masking and online softmax (base 2)
    const bool unit_masked = !b_ok || (pa + 2) * kPage > L;
    float x[8];
    bool valid[8];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = (pa + pg) * kPage + 4 * q4 + i;
        const bool ok = head_ok && (pg == 0 || b_ok) && tok < L;
        valid[4 * pg + i] = (pg == 0 || b_ok) && tok < L;
        x[4 * pg + i] = ok ? sc[pg][i] * cmul : -INFINITY;
      }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = (m_new == m_run) ? 1.0f : exp2f(m_run - m_use);
    float p[8];
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(x[e] - m_use);
      psum += p[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * q4 + i);
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[jt][i] *= ar[i];
    }

    // ---- P.V
    if constexpr (I8) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        h8_t phi, plo;
#pragma unroll
        for (int pg = 0; pg < 2; ++pg)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * pg + i;
            const float sv = valid[e] ? scale_at(pg ? vsB : vsA, i * NG + g) : 0.0f;
            const float pp = p[e] * sv;
            const _Float16 hi = (_Float16)pp;
            phi[e] = hi;
            plo[e] = (_Float16)fmaf(p[e], sv, -(float)hi);
          }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int jt = 2 * g + jj;
          const h8_t bv = i8x8_to_h8(vA[jt >> 2][jt & 3], vB[jt >> 2][jt & 3]);
          acc[jt] = mfma_f16(phi, bv, acc[jt]);
          acc[jt] = mfma_f16(plo, bv, acc[jt]);
        }
      }
    } else {
      b8_t phi, plo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 hi = (__bf16)p[e];
        phi[e] = hi;
        plo[e] = (__bf16)(p[e] - (float)hi);
      }
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        u4_t w = {vA[jt >> 1][(jt & 1) * 2], vA[jt >> 1][(jt & 1) * 2 + 1], vB[jt >> 1][(jt & 1) * 2],
                  vB[jt >> 1][(jt & 1) * 2 + 1]};
        if (unit_masked) {  // unwritten slots may hold any bits (NaN): zero them
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!valid[e]) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        const b8_t bv = __builtin_bit_cast(b8_t, w);
        acc[jt] = mfma_bf16(phi, bv, acc[jt]);
        acc[jt] = mfma_bf16(plo, bv, acc[jt]);
      }
    }
  }

  // ---- per-head sum over the four lane rows
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  const int64_t row0 = ((int64_t)s * a.Hq + (int64_t)h * G) * a.NS + j;  // partial of head h*G + 0
  if constexpr (NW == 1) {
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 4 * q4 + i;
        if (hh < G) a.o_part[(row0 + (int64_t)hh * a.NS) * D + 16 * jt + n16] = acc[jt][i];
      }
    if (q4 == 0 && head_ok) a.ml[row0 + (int64_t)n16 * a.NS] = make_float2(m_run, l_run);
  } else {
    extern __shared__ float smem[];
    float *s_acc = smem;                 // [NW][G][D]
    float *s_m = smem + NW * G * D;      // [NW][16]
    float *s_l = s_m + NW * 16;          // [NW][16]
    if (q4 == 0) {
      s_m[wave * 16 + n16] = m_run;
      s_l[wave * 16 + n16] = l_run;
    }
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 4 * q4 + i;
        if (hh < G) s_acc[(wave * G + hh) * D + 16 * jt + n16] = acc[jt][i];
      }
    __syncthreads();
    for (int e = threadIdx.x; e < G * D; e += NW * 64) {
      const int hh = e / D, c = e - hh * D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w * 16 + hh]);
      float o = 0.0f, l = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = s_m[w * 16 + hh];
        if (mw != -INFINITY) {
          const float wt = exp2f(mw - M);
          o = fmaf(wt, s_acc[(w * G + hh) * D + c], o);
          l = fmaf(wt, s_l[w * 16 + hh], l);
        }
      }
      a.o_part[(row0 + (int64_t)hh * a.NS) * D + c] = o;
      if (c == 0) a.ml[row0 + (int64_t)hh * a.NS] = make_float2(M, l);
    }
  }
}

// ------------------------------------------------------------------ decode: merge
//
// Workgroup (64-channel chunk, query head, sequence) of 4 wavefronts; wave w takes splits
// w, w+4, ...  M = max_j m_j over the splits that hold pages; w_j = 2^(m_j - M);
// out = sum_j w_j o_j / sum_j w_j l_j; lse = ln 2 * (M + log2 sum_j w_j l_j).
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int NCH = D / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x % NCH;
  const int hq = (blockIdx.x / NCH) % a.Hq;
  const int s = blockIdx.x / (NCH * a.Hq);
  int L = a.context_lens[s];
  L = max(0, min(L, a.max_context_len));
  const int P = (L + kPage - 1) / kPage;
  const int nsa = min(a.NS, (P + a.cpp - 1) / a.cpp);
  const int c = chunk * 64 + lane;
  const int64_t orow = ((int64_t)s * a.Hq + hq);
  if (nsa == 0) {
    if (wave == 0) {
      a.out[orow * D + c] = 0.0f;
      if (a.lse && chunk == 0 && lane == 0) a.lse[orow] = -INFINITY;
    }
    return;
  }
  const int64_t base = orow * a.NS;
  float M = -INFINITY;
  for (int jj = lane; jj < nsa; jj += 64) M = fmaxf(M, a.ml[base + jj].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float o = 0.0f, l = 0.0f;
  for (int jj = wave; jj < nsa; jj += 4) {
    const float2 ml = a.ml[base + jj];
    if (ml.x != -INFINITY) {
      const float w = exp2f(ml.x - M);
      o = fmaf(w, a.o_part[(base + jj) * D + c], o);
      l = fmaf(w, ml.y, l);
    }
  }
  __shared__ float s_o[4][64];
  __shared__ float s_l[4];
  s_o[wave][lane] = o;
  if (lane == 0) s_l[wave] = l;
  __syncthreads();
  if (wave == 0) {
    const float ot = s_o[0][lane] + s_o[1][lane] + s_o[2][lane] + s_o[3][lane];
    const float lt = s_l[0] + s_l[1] + s_l[2] + s_l[3];
    a.out[orow * D + c] = ot / lt;
    if (a.lse && chunk == 0 && lane == 0) a.lse[orow] = kLn2 * (M + log2f(lt));
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_kv_write(int dtype, const WriteArgs &a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int per = (dtype == 0 ? a.D / kGroup : a.D / 8) * 2;
  const int64_t total = (int64_t)a.T * a.Hkv * per;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (dtype == 0) {
    if (a.D == 256) hipLaunchKernelGGL(kv_write_i8_kernel<256>, dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(kv_write_i8_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (a.D == 256) hipLaunchKernelGGL(kv_write_bf16_kernel<256>, dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(kv_write_bf16_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D, int NW, bool I8>
static void launch_split(const DecodeArgs &a, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.S * a.Hkv * a.NS);
  const size_t smem = NW > 1 ? (size_t)(NW * a.G * D + NW * 32) * sizeof(float) : 0;
  hipLaunchKernelGGL((decode_split_kernel<D, NW, I8>), dim3(grid), dim3(NW * 64), smem, stream, a);
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

hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t stream) {
  if (dtype == 0) {
    if (a.D == 256) launch_split_nw<256, true>(a, stream);
    else launch_split_nw<128, true>(a, stream);
  } else {
    if (a.D == 256) launch_split_nw<256, false>(a, stream);
    else launch_split_nw<128, false>(a, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((int64_t)a.S * a.Hq * (a.D / 64));
  if (a.D == 256) hipLaunchKernelGGL(decode_merge_kernel<256>, dim3(grid), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
