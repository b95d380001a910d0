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
// LPR lanes (an aligned group of a wave) own a row: lane l of the group holds the 16 / LPR groups
// of eight consecutive elements 8 (l + LPR k) .. 8 (l + LPR k) + 7, k < 16 / LPR, so that for
// each k the group's lanes hold one contiguous piece of the row (one coalesced 16-byte load per
// lane). The arithmetic is compiled without FP contraction so codes and scales are bit-identical
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

// Cross-lane butterfly stage h = 8 M (partner lane l ^ M): the lane holding the lower element of
// each pair keeps a + b, its partner a - b. The partner negates its own value first, so both lanes
// add: other + (-b) is exactly a - b in IEEE arithmetic, and b + a exactly a + b.
template <int M, int K>
__device__ __forceinline__ void fwht_cross(float (&r)[K][8], int l) {
  const uint32_t neg = (l & M) ? 0x80000000u : 0u;
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float mine = __uint_as_float(__float_as_uint(r[k][e]) ^ neg);
      r[k][e] = shfl_xor16<M>(r[k][e]) + mine;
    }
}

template <int M>
__device__ __forceinline__ float max_xor(float v) {
  return fmaxf(v, shfl_xor16<M>(v));
}

// Unnormalised FWHT of the row in stage order h = 1, 2, ..., 64: element 8 (l + LPR k) + e sits
// in r[k][e] of lane l, so stages 1..4 pair elements of one lane's group, stages 8 .. 4 LPR pair
// lanes, and stages 8 LPR .. 64 pair groups k of one lane.
template <int LPR>
__device__ __forceinline__ void fwht_row(float (&r)[16 / LPR][8], int l) {
#pragma clang fp contract(off)
  constexpr int K = 16 / LPR;
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((e & h) == 0) {
          const float a = r[k][e], b = r[k][e + h];
          r[k][e] = a + b;
          r[k][e + h] = a - b;
        }
  if constexpr (LPR >= 2) fwht_cross<1>(r, l);
  if constexpr (LPR >= 4) fwht_cross<2>(r, l);
  if constexpr (LPR >= 8) fwht_cross<4>(r, l);
  if constexpr (LPR >= 16) fwht_cross<8>(r, l);
#pragma unroll
  for (int m = 1; m < K; m <<= 1)
#pragma unroll
    for (int k = 0; k < K; ++k)
      if ((k & m) == 0)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = r[k][e], b = r[k + m][e];
          r[k][e] = a + b;
          r[k + m][e] = a - b;
        }
}

// Eight codes (their low bits) packed little-endian into one 8 BITS-bit field.
template <int BITS>
__device__ __forceinline__ uint32_t pack8(const uint32_t (&c)[8]) {
  constexpr uint32_t mask = (1u << BITS) - 1u;
  if constexpr (BITS == 4) {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = ((c[2 * i + 1] << 4) | (c[2 * i] & mask)) & 0xffu;
    return p[0] | (p[1] << 8) | (p[2] << 16) | (p[3] << 24);
  } else {
    static_assert(BITS == 2 || BITS == 3, "turbo8 packs bytes");
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) w |= (c[e] & mask) << (BITS * e);
    return w;
  }
}

// The row's codes from the transform output x (unscaled), packed: w[k][0] holds group k's field
// (8 BITS bits; turbo8 uses w[k][0] and w[k][1], four bytes each). The definition is
// c = clamp(rint(fl(fl(x C) / s16)), +-qmax), 0 when s16 = 0. For turbo4/3/2 (qmax <= 7) the
// quotient is first taken as y = x * fl(C * rcp(s16)): the hardware reciprocal is within one ulp,
// so |y - fl(fl(x C) / s16)| <= (qmax + 1/4) * 2^-21.4 < 2^-18 whenever the row's largest |y| is
// below qmax + 1/4, and rint(y) (taken by adding 1.5 * 2^23, whose sum holds the integer in its
// low mantissa bits) is the exact code unless y lies within 2^-16 of a half-integer. A lane where
// that can fail (a near tie, a large or non-finite |y|) recomputes its codes with IEEE division.
template <int BITS, int K>
__device__ __forceinline__ void quantize_pack(const float (&x)[K][8], float xmax, float sf, uint32_t (&w)[K][2]) {
#pragma clang fp contract(off)
  constexpr int qmax = (1 << (BITS - 1)) - 1;
  bool exact = true;
  if constexpr (qmax <= 7) {
    constexpr float kMagic = 0x1.8p23f;
    constexpr float kEps = 0x1p-16f;
    const float kq = sf != 0.f ? kRotC * __builtin_amdgcn_rcpf(sf) : 0.f;
    bool redo = !(xmax * kq < (float)qmax + 0.25f);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = x[k][e] * kq;
        const float m = y + kMagic;
        const float d = (m - kMagic) - y;
        redo |= !(fabsf(d) < 0.5f - kEps);
        c[e] = __float_as_uint(m);
      }
      w[k][0] = pack8<BITS>(c);
      w[k][1] = 0u;
    }
    exact = redo;
  }
  if (exact) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float q = fminf(fmaxf(rintf((x[k][e] * kRotC) / sf), (float)-qmax), (float)qmax);
        c[e] = (uint32_t)(int)(sf != 0.f ? q : 0.f);   // (a select: no branch per element)
      }
      if constexpr (BITS == 8) {
        w[k][0] = (c[0] & 0xffu) | ((c[1] & 0xffu) << 8) | ((c[2] & 0xffu) << 16) | (c[3] << 24);
        w[k][1] = (c[4] & 0xffu) | ((c[5] & 0xffu) << 8) | ((c[6] & 0xffu) << 16) | (c[7] << 24);
      } else {
        w[k][0] = pack8<BITS>(c);
        w[k][1] = 0u;
      }
    }
  }
}

// Encode one row: raw[k] = this lane's eight bf16 elements 8 (l + LPR k) .. + 7; block = the
// (page, kv head) block, slot = the token's slot in the page.
template <int BITS, int LPR>
__device__ __forceinline__ void encode_row_lanes(const uint4 (&raw)[16 / LPR], int l, uint8_t* block, int slot,
                                                 int page_size) {
#pragma clang fp contract(off)
  constexpr int K = 16 / LPR;
  if constexpr (BITS == 0) {
    // unquantized cache: copy the bf16 row into its slot
#pragma unroll
    for (int k = 0; k < K; ++k)
      *reinterpret_cast<uint4*>(block + (int64_t)slot * 256 + (l + LPR * k) * 16) = raw[k];
    return;
  } else if constexpr (BITS == kFp8) {
    // fp8 cache: eight E4M3 bytes per group
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b0 = fp8_e4m3(bf16_lo(w[e])), b1 = fp8_e4m3(bf16_hi(w[e]));
        const uint32_t pair = b0 | (b1 << 8);
        if (e < 2) lo |= pair << (16 * e);
        else hi |= pair << (16 * (e - 2));
      }
      *reinterpret_cast<uint2*>(block + (int64_t)slot * 128 + (l + LPR * k) * 8) = make_uint2(lo, hi);
    }
    return;
  } else {
    constexpr int qmax = (1 << (BITS - 1)) - 1;
    float r[K][8];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      r[k][0] = bf16_lo(raw[k].x);
      r[k][1] = bf16_hi(raw[k].x);
      r[k][2] = bf16_lo(raw[k].y);
      r[k][3] = bf16_hi(raw[k].y);
      r[k][4] = bf16_lo(raw[k].z);
      r[k][5] = bf16_hi(raw[k].z);
      r[k][6] = bf16_lo(raw[k].w);
      r[k][7] = bf16_hi(raw[k].w);
    }
    fwht_row<LPR>(r, l);
    // absmax of the rotated row: max |fl(x C)| = fl(max |x| * C), rounding being monotonic
    // (NaN elements are passed over, as by fmaxf)
    float xm = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) xm = fmaxf(xm, fabsf(r[k][e]));
    if constexpr (LPR >= 2) xm = max_xor<1>(xm);
    if constexpr (LPR >= 4) xm = max_xor<2>(xm);
    if constexpr (LPR >= 8) xm = max_xor<4>(xm);
    if constexpr (LPR >= 16) xm = max_xor<8>(xm);
    const float amax = xm * kRotC;
    const float s32 = amax / (float)qmax;
    const _Float16 s16 = (_Float16)fminf(s32, 65504.f);
    const float sf = (float)s16;
    uint32_t pw[K][2];
    quantize_pack<BITS, K>(r, xm, sf, pw);

    constexpr int rowb = 16 * BITS;
    uint8_t* dst = block + (int64_t)slot * rowb;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int grp = l + LPR * k;   // group of eight elements within the row
      if constexpr (BITS == 8) {
        *reinterpret_cast<uint2*>(dst + 8 * grp) = make_uint2(pw[k][0], pw[k][1]);
      } else if constexpr (BITS == 4) {
        *reinterpret_cast<uint32_t*>(dst + 4 * grp) = pw[k][0];
      } else if constexpr (BITS == 2) {
        *reinterpret_cast<uint16_t*>(dst + 2 * grp) = (uint16_t)pw[k][0];
      } else {
        // BITS == 3: 24 bits per group at bit offset 24 grp. The LPR groups of one k are
        // contiguous (3 LPR / 4 dwords); dword j of them starts in group (32 j) / 24 at bit
        // (32 j) mod 24, so lane j < 3 LPR / 4 joins its group's field with the next lane's.
        const uint32_t v = pw[k][0];
        const int src = (32 * l) / 24, off = (32 * l) % 24;
        uint32_t lo, hi;
        if constexpr (LPR == 4) {
          // lane l takes lanes l (l < 3: src = l) and l + 1 of its quad (DPP quad_perm [1,2,3,3])
          lo = v;
          hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xF9, 0xF, 0xF, true);
        } else {
          const int base = (threadIdx.x & 63) & ~(LPR - 1);
          lo = (uint32_t)__shfl((int)v, base + min(src, LPR - 1), 64);
          hi = (uint32_t)__shfl((int)v, base + min(src + 1, LPR - 1), 64);
        }
        const uint32_t wd = (lo >> off) | (hi << (24 - off));
        if (l < 3 * LPR / 4) *reinterpret_cast<uint32_t*>(dst + 3 * LPR * k + 4 * l) = wd;
      }
    }
    if (l == 0) {
      uint16_t* sdst = reinterpret_cast<uint16_t*>(block + (int64_t)page_size * rowb) + slot;
      *sdst = __builtin_bit_cast(uint16_t, s16);
    }
  }
}

// The passes of an append: four lanes a row, 16 rows a pass, one kv head of 16 consecutive
// tokens (a chunk's consecutive positions fill consecutive slots of a page, so a pass writes one
// run of codes and one of scales per page). Passes 0 .. npass - 1 encode K rows, npass ..
// 2 npass - 1 V rows; the calling wave runs passes first, first + stride, ..., each with the next
// one's rows already loading (the rows are streamed once: non-temporal loads).
constexpr int kAppendLanes = 4;
constexpr int kAppendRows = 64 / kAppendLanes;

template <int BITS>
__device__ __forceinline__ void append_passes(const AppendParams& p, uint32_t first, uint32_t stride, int lane) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  struct RowIn {
    uint4 raw[kAppendLanes];   // this lane's four pieces
    int seq, pos;              // the row's token: its sequence and position
  };
  const int l = lane & (kAppendLanes - 1);      // lane of the row
  const int rw = lane / kAppendLanes;           // token of the pass's 16
  const uint32_t ntok = (uint32_t)p.n_tokens;   // n_tokens * hkv < 2^28, checked by the caller
  const uint32_t hkv = (uint32_t)p.hkv;
  const uint32_t npass = (ntok + kAppendRows - 1) / kAppendRows * hkv;   // 16-token block x kv head
  const int shift = __builtin_ctz((unsigned)p.page_size);

  auto token_of = [&](uint32_t pass) { return (pass % npass) / hkv * kAppendRows + rw; };
  auto load = [&](uint32_t pass, RowIn& in) __attribute__((always_inline)) {
    const uint32_t tok = token_of(pass);
    if (tok < ntok) {
      const uint32_t row = tok * hkv + (pass % npass) % hkv;
      const uint16_t* s = (pass < npass ? p.k_new : p.v_new) + (int64_t)row * kHeadDim + 8 * l;
#pragma unroll
      for (int k = 0; k < kAppendLanes; ++k) {
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(s + 8 * kAppendLanes * k));
        in.raw[k] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      in.seq = p.token_seq[tok];
      in.pos = p.token_pos[tok];
    }
  };

  uint32_t pass = first;
  RowIn cur;
  if (pass < 2 * npass) load(pass, cur);
  while (pass < 2 * npass) {
    const uint32_t tok = token_of(pass);
    const uint32_t head = (pass % npass) % hkv;
    int page = 0;
    if (tok < ntok) page = p.block_tables[(int64_t)cur.seq * p.maxp + (cur.pos >> shift)];
    const uint32_t next = pass + stride;
    RowIn nxt;
    if (next < 2 * npass) load(next, nxt);
    if (tok < ntok) {
      uint8_t* block = (pass < npass ? p.k_pool : p.v_pool) + (int64_t)page * p.page_stride +
                       (int64_t)head * p.block_bytes;
      encode_row_lanes<BITS, kAppendLanes>(cur.raw, l, block, cur.pos & (p.page_size - 1), p.page_size);
    }
    cur = nxt;
    pass = next;
  }
}

// Sixteen lanes per row, one group each (the fused append + decode path).
template <int BITS>
__device__ __forceinline__ void encode_row(const uint4 raw, int lane16, uint8_t* block, int slot, int page_size) {
  const uint4 g[1] = {raw};
  encode_row_lanes<BITS, 16>(g, lane16, block, slot, page_size);
}

}  // namespace codec
}  // namespace xq
