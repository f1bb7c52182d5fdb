// Device-side helpers shared by the gfx950 kernels of libdg.
//
// Numeric conventions (the FP8 block-quantised GEMM page on lpnh.cn, s2.2,
// s3.1, s4.2): FP8 is E4M3 with bias 7, no infinities and largest finite value
// 448; rounding is to nearest, ties to even; BF16 outputs are rounded to
// nearest-even from FP32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.hpp"

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Two FP32 values rounded to BF16 (nearest, ties to even), packed: a in the
// low half, b in the high half.  One v_cvt_pk_bf16_f32 on gfx950; an
// exhaustive sweep of all 2^32 binary32 inputs on the GPU matched the
// integer rounding (u + 0x7FFF + lsb) >> 16 bit for bit on every finite
// input, normal and subnormal, and kept NaN a NaN (the integer form can
// turn a NaN into infinity).  It replaces about ten VALU instructions per
// pair in every epilogue: staging a 256 x 256 tile through LDS went from
// ~4.7k to ~2.7k cycles (the conversion had made it VALU-bound).
typedef float dg_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 dg_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((dg_f2){a, b}, dg_bf16x2));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float half_wave_max(float v) {
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ---- E4M3 block encoding, shared by the quantiser and the GEMM that
// quantises its activations on the fly (FP8 block-quantised GEMM page on
// lpnh.cn, s4.2 steps 3-4 and the RNE note; s5.4 for all-zero blocks) ----

// Per-block scale s = amax / 448 (one binary32 division; the stored scale)
// and what the quotients x / s are formed from: k = 1, or 2^64 when s < 2^-62
// (sk = s k and x k are then exact, so (x k) / sk = x / s), and r = RN(1/sk)
// (0 for an all-zero block, s = 0).
struct BlockScale {
  float s, k, sk, r;
};

__device__ __forceinline__ BlockScale block_scale(float amax) {
  BlockScale b;
  b.s = amax / 448.0f;
  b.k = b.s < 0x1p-62f ? 0x1p64f : 1.0f;
  b.sk = b.s * b.k;
  b.r = b.s == 0.0f ? 0.0f : 1.0f / b.sk;
  return b;
}

// Correctly rounded binary32 quotient x / s from r = RN(1/s) and one FMA
// correction (Markstein: q = RN(x r), q' = RN(q + (x - q s) r) = RN(x/s)
// provided the remainder x - q s is exact).  The remainder is a multiple of
// ulp(q) ulp(s); for quotients >= 2^-11 (smaller ones encode to zero either
// way) and s >= 2^-62 that is >= 2^-119, inside binary32's range, so the
// remainder is representable.  Smaller scales, subnormal ones included, are
// lifted by 2^64 first (block_scale).
__device__ __forceinline__ float quotient_rn(float x, float s, float r) {
  const float q = x * r;
  const float e = __builtin_fmaf(-q, s, x);
  return __builtin_fmaf(e, r, q);
}

// |x| / s, correctly rounded, capped at 448.  The quotient is formed on |x|
// (s > 0, so |x/s| = |x|/s) and the sign bit is restored by the caller: the
// FMA correction would turn a -0 quotient into +0.  Quotients above 448 round
// to 448 in E4M3 anyway (saturation).  In an all-zero block (sk = r = 0)
// every step yields 0.
__device__ __forceinline__ float magnitude_quotient(float x, const BlockScale& b) {
  return fminf(quotient_rn(fabsf(x) * b.k, b.sk, b.r), 448.0f);
}

// Sign bits of four values placed at bit 7 of each code byte.
__device__ __forceinline__ uint32_t zero_codes4(float4 v) {
  return ((__float_as_uint(v.x) >> 31) << 7) | ((__float_as_uint(v.y) >> 31) << 15) |
         ((__float_as_uint(v.z) >> 31) << 23) | ((__float_as_uint(v.w) >> 31) << 31);
}

// Codes of four values of a block with scale b: round to the nearest E4M3
// code, ties to even, with v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950, default
// round-to-nearest-even mode), then OR in the sign bits.  The instruction's
// result was compared on an MI355X with a ties-to-even encoder written from
// the E4M3 field layout, for every binary32 magnitude below 464 and both
// signs (including binary32 subnormals and -0): no difference.  Branch-free.
__device__ __forceinline__ uint32_t encode4_block(float4 v, const BlockScale& b) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(magnitude_quotient(v.x, b), magnitude_quotient(v.y, b),
                                          0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(magnitude_quotient(v.z, b), magnitude_quotient(v.w, b), p,
                                      true);
  return (uint32_t)p | zero_codes4(v);
}

// ---- power-of-two (UE8M0) block scales (DeepGEMM page on pzsr.cn, s3.1:
// UE8M0 scaling factors, four per 32-bit word) ----

// Smallest E in [0, 254] with 2^(E - 127) >= t (t >= 0 finite): t rounded up
// to a power of two, as a UE8M0 byte.  Subnormal t = m 2^-149 needs E = 1
// only when m > 2^22 (t > 2^-127); t = 0 gives 0.
__device__ __forceinline__ int ue8m0_exponent(float t) {
  const uint32_t u = __float_as_uint(t);
  const int ex = (int)(u >> 23);
  const uint32_t m = u & 0x7FFFFFu;
  if (ex == 0) return m > 0x400000u ? 1 : 0;
  const int e = ex + (m != 0u ? 1 : 0);
  return e > 254 ? 254 : e;
}

// 2^n as binary32 for n in [-127, 127] (2^-127 is subnormal).
__device__ __forceinline__ float pow2f(int n) {
  return n >= -126 ? __uint_as_float((uint32_t)(n + 127) << 23) : __uint_as_float(0x00400000u);
}

// Encoder parameters for the scale 2^(E - 127): the quotient x / s is the
// exact product x * 2^(127 - E) (rounded only when it falls below binary32's
// normal range, far under the smallest E4M3 subnormal), so no rescaling.
__device__ __forceinline__ BlockScale pow2_block_scale(int e) {
  BlockScale b;
  b.s = pow2f(e - 127);
  b.k = 1.0f;
  b.sk = b.s;
  b.r = pow2f(127 - e);
  return b;
}

__device__ __forceinline__ float abs_max4(float m, float4 v) {
  return fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Maximum over each row of 16 lanes (lanes 16i .. 16i+15), with DPP moves:
// swap neighbours, swap pairs, mirror each half-row, mirror the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// Maximum over aligned groups of G consecutive lanes (G = 4, 8 or 16): the
// first two, three or four moves of row16_max.
template <int G>
__device__ __forceinline__ float lane_group_max(float v) {
  static_assert(G == 4 || G == 8 || G == 16, "lane group");
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  if constexpr (G >= 8)
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  if constexpr (G >= 16)
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// ---- fused epilogue (bjdmk.com.cn DeepGEMM page, s3.2: activation and
// residual applied while the product is in registers; pzsr.cn page, s2.3:
// SwiGLU), in FP32 before the BF16 rounding ----

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + expf(-v)); }

__device__ __forceinline__ float act_f(float v, int act) {
  switch (act) {
    case EPI_RELU: return v > 0.0f ? v : 0.0f;
    case EPI_SILU: return silu_f(v);
    case EPI_GELU: return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
    default: return v;
  }
}

template <int V>
struct IntTag {
  static constexpr int value = V;
};

// f(IntTag<0>{}) ... f(IntTag<N-1>{}), unrolled at compile time.
template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F&& f) {
  if constexpr (I < N) {
    f(IntTag<I>{});
    static_for_from<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_from<0, N>(f);
}

// As static_for, but stops after the first call that returns false.
template <int I, int N, class F>
__device__ __forceinline__ void static_while_from(F&& f) {
  if constexpr (I < N) {
    if (f(IntTag<I>{})) static_while_from<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_while(F&& f) {
  static_while_from<0, N>(f);
}

// The results t[0..3] of columns n .. n+3 (n % 4 == 0) of row m after the
// epilogue ACT (an EpiAct; SwiGLU pairs the columns: 2j gate, 2j+1 up ->
// output column j), then the residual if RES, then BF16 round-to-nearest-
// even.  Returns the number of output columns (4, or 2 for SwiGLU, packed in
// v.x); the first one is column n, or n / 2 for SwiGLU.
template <int ACT, bool RES>
__device__ __forceinline__ int epilogue4(int64_t m, int64_t n, const float* t, const Epilogue& e,
                                         uint2& v) {
  if constexpr (ACT == EPI_SWIGLU) {
    float o0 = silu_f(t[0]) * t[1];
    float o1 = silu_f(t[2]) * t[3];
    if constexpr (RES) {
      const uint32_t r = *reinterpret_cast<const uint32_t*>(e.res + m * e.ldc + (n >> 1));
      o0 += bf16_bits_to_f32(r & 0xFFFFu);
      o1 += bf16_bits_to_f32(r >> 16);
    }
    v.x = bf16x2_rne(o0, o1);
    v.y = 0;
    return 2;
  } else {
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = act_f(t[r], ACT);
    if constexpr (RES) {
      const uint2 r = *reinterpret_cast<const uint2*>(e.res + m * e.ldc + n);
      o[0] += bf16_bits_to_f32(r.x & 0xFFFFu);
      o[1] += bf16_bits_to_f32(r.x >> 16);
      o[2] += bf16_bits_to_f32(r.y & 0xFFFFu);
      o[3] += bf16_bits_to_f32(r.y >> 16);
    }
    v.x = bf16x2_rne(o[0], o[1]);
    v.y = bf16x2_rne(o[2], o[3]);
    return 4;
  }
}

// epilogue4, written straight to C [.][ldc].
template <int ACT, bool RES>
__device__ __forceinline__ void store4(uint16_t* c, int64_t m, int64_t n, const float* t,
                                       const Epilogue& e) {
  uint2 v;
  if (epilogue4<ACT, RES>(m, n, t, e, v) == 2)
    *reinterpret_cast<uint32_t*>(c + m * e.ldc + (n >> 1)) = v.x;
  else
    *reinterpret_cast<uint2*>(c + m * e.ldc + n) = v;
}

// Runs f(IntTag<ACT>, IntTag<RES>) for the epilogue e, choosing the variant
// once per store loop: with the choice made per element, every store site
// carries every variant inline and the epilogue path sprawls over the
// instruction cache (measured: ~16 us more per 256 x 256 tile).
template <class F>
__device__ __forceinline__ void with_epilogue(const Epilogue& e, F&& f) {
  const bool r = e.res != nullptr;
  switch (e.act) {
    case EPI_RELU:
      if (r) f(IntTag<EPI_RELU>{}, IntTag<1>{}); else f(IntTag<EPI_RELU>{}, IntTag<0>{});
      break;
    case EPI_SILU:
      if (r) f(IntTag<EPI_SILU>{}, IntTag<1>{}); else f(IntTag<EPI_SILU>{}, IntTag<0>{});
      break;
    case EPI_GELU:
      if (r) f(IntTag<EPI_GELU>{}, IntTag<1>{}); else f(IntTag<EPI_GELU>{}, IntTag<0>{});
      break;
    case EPI_SWIGLU:
      if (r) f(IntTag<EPI_SWIGLU>{}, IntTag<1>{}); else f(IntTag<EPI_SWIGLU>{}, IntTag<0>{});
      break;
    default:
      if (r) f(IntTag<EPI_NONE>{}, IntTag<1>{}); else f(IntTag<EPI_NONE>{}, IntTag<0>{});
      break;
  }
}

}  // namespace dg
