// Encoding of one K or V row into its cache slot, shared by the append kernel and the fused
// append + decode path (both must write the same bytes).
//
// Method: "xInfer: Pure-Rust LLM Inference Without a Python Runtime" (hysenlabs.com), section
// "What actually sits between the request and the tokens": the row is rotated by a
// Walsh-Hadamard transform and quantized with a per-head absmax scale. Number format fixed by
// this library (the pages leave it open): fp32 FWHT stages h = 1..64 of (a+b, a-b), one multiply
// by C = fp32(1/sqrt(128)), s16 = fp16_rne(min(absmax/qmax, 65504)), c = clamp(rint_half_even(
// x/s16), +-qmax), bits-wide two's complement fields packed little-endian. fp8 (same page,
// section "Getting a server up: the commands in the README"): the nearest finite OCP E4M3 value of
// each element, ties to even, saturating at 448; bf16: the row as it is.
//
// Sixteen lanes own a row (an aligned group of 16 lanes of a wave), eight consecutive elements
// each. The arithmetic is compiled without FP contraction so codes and scales are bit-identical
// to the CPU definition.
#pragma once

#include "xq_internal.h"

namespace xq {
namespace codec {

constexpr float kRotC = 0x1.6a09e6p-4f;   // fp32 nearest to 1/sqrt(128), bits 0x3DB504F3

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// OCP FP8 E4M3 byte of a finite fp32 value: sign kept; magnitudes from 448 on give 448 (0x7E);
// normal results (from 2^-6) keep 3 mantissa bits rounded to nearest, ties to even, where a
// carry moves into the exponent; below 2^-6 the result is the nearest multiple of 2^-9
// (subnormal codes 0..7, or 8 = 2^-6), rounded half to even.
__device__ __forceinline__ uint32_t fp8_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t c;
  if (a >= 0x43e00000u) {              // 448
    c = 0x7eu;
  } else if (a >= 0x3c800000u) {       // 2^-6
    c = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  } else {
    c = (uint32_t)rintf(__uint_as_float(a) * 512.f);
  }
  return sign | c;
}

// Value held by lane (lane ^ M) of the 16-lane group that owns a row: DPP quad_perm (M = 1, 2)
// and row_ror:8 (M = 8, a row being 16 lanes) are VALU operand modifiers, M = 4 a ds_swizzle in
// bit-mask mode (no memory access). Pure data movement: the arithmetic is unchanged.
template <int M>
__device__ __forceinline__ float shfl_xor16(float v) {
  if constexpr (M == 1 || M == 2) {
    constexpr int kCtrl = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] and [2,3,0,1]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
  } else if constexpr (M == 8) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true));
  } else {
    static_assert(M == 4, "exchanges within 16 lanes");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
  }
}

template <int M>
__device__ __forceinline__ void fwht_cross(float (&r)[8], int lane16) {
  const bool upper = (lane16 & M) != 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float other = shfl_xor16<M>(r[e]);
    r[e] = upper ? (other - r[e]) : (r[e] + other);
  }
}

// Encode one row: raw = this lane's eight bf16 elements (8 lane16 .. 8 lane16 + 7); block = the
// (page, kv head) block, slot = the token's slot in the page.
template <int BITS>
__device__ __forceinline__ void encode_row(const uint4 raw, int lane16, uint8_t* block, int slot, int page_size) {
#pragma clang fp contract(off)
  if constexpr (BITS == 0) {
    // unquantized cache: copy the bf16 row into its slot
    *reinterpret_cast<uint4*>(block + (int64_t)slot * 256 + lane16 * 16) = raw;
    return;
  } else if constexpr (BITS == kFp8) {
    // fp8 cache: eight E4M3 bytes per lane, elements 8 lane16 .. 8 lane16 + 7
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t b0 = fp8_e4m3(bf16_lo(w[e])), b1 = fp8_e4m3(bf16_hi(w[e]));
      const uint32_t pair = b0 | (b1 << 8);
      if (e < 2) lo |= pair << (16 * e);
      else hi |= pair << (16 * (e - 2));
    }
    *reinterpret_cast<uint2*>(block + (int64_t)slot * 128 + lane16 * 8) = make_uint2(lo, hi);
    return;
  } else {
    constexpr int qmax = (1 << (BITS - 1)) - 1;
    float r[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                  bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
    // in-lane stages h = 1, 2, 4 (element index 8*lane16 + e)
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((e & h) == 0) {
          const float a = r[e], b = r[e + h];
          r[e] = a + b;
          r[e + h] = a - b;
        }
      }
    }
    // cross-lane stages h = 8, 16, 32, 64: the lane with bit (h/8) clear holds the lower
    // element of every pair and keeps a + b; its partner keeps a - b.
    fwht_cross<1>(r, lane16);
    fwht_cross<2>(r, lane16);
    fwht_cross<4>(r, lane16);
    fwht_cross<8>(r, lane16);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      r[e] = r[e] * kRotC;
      amax = fmaxf(amax, fabsf(r[e]));
    }
    amax = fmaxf(amax, shfl_xor16<1>(amax));
    amax = fmaxf(amax, shfl_xor16<2>(amax));
    amax = fmaxf(amax, shfl_xor16<4>(amax));
    amax = fmaxf(amax, shfl_xor16<8>(amax));

    const float s32 = amax / (float)qmax;
    const _Float16 s16 = (_Float16)fminf(s32, 65504.f);
    const float sf = (float)s16;
    int code[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c = 0.f;
      if (sf != 0.f) c = fminf(fmaxf(rintf(r[e] / sf), (float)-qmax), (float)qmax);
      code[e] = (int)c;
    }

    constexpr int rowb = 16 * BITS;
    uint8_t* dst = block + (int64_t)slot * rowb;
    if constexpr (BITS == 4) {
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) w |= (uint32_t)(code[e] & 0xf) << (4 * e);
      *reinterpret_cast<uint32_t*>(dst + 4 * lane16) = w;
    } else if constexpr (BITS == 8) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0 |= (uint32_t)(code[e] & 0xff) << (8 * e);
        w1 |= (uint32_t)(code[e + 4] & 0xff) << (8 * e);
      }
      *reinterpret_cast<uint2*>(dst + 8 * lane16) = make_uint2(w0, w1);
    } else if constexpr (BITS == 2) {   // 16 bits per lane, two bytes
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) w |= (uint32_t)(code[e] & 0x3) << (2 * e);
      *reinterpret_cast<uint16_t*>(dst + 2 * lane16) = (uint16_t)w;
    } else {  // BITS == 3: 24 bits per lane at bit offset 24*lane16; 12 dwords per row
      uint32_t v = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) v |= (uint32_t)(code[e] & 0x7) << (3 * e);
      // dword k of the row starts in lane (32k)/24 at bit offset 32k mod 24
      const int k = lane16;
      const int src_lane = (32 * k) / 24;
      const int off = (32 * k) % 24;
      const int base = threadIdx.x & ~15;
      const uint32_t lo = (uint32_t)__shfl((int)v, base + min(src_lane, 15), 64);
      const uint32_t hi = (uint32_t)__shfl((int)v, base + min(src_lane + 1, 15), 64);
      const uint32_t w = (lo >> off) | (hi << (24 - off));
      if (k < 12) *reinterpret_cast<uint32_t*>(dst + 4 * k) = w;
    }
    if (lane16 == 0) {
      uint16_t* sdst = reinterpret_cast<uint16_t*>(block + (int64_t)page_size * rowb) + slot;
      *sdst = __builtin_bit_cast(uint16_t, s16);
    }
  }
}

}  // namespace codec
}  // namespace xq
