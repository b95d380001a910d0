// Paged single-token decode attention over a TurboQuant (or bf16) KV cache, gfx950.
//
// Method: "xInfer: Pure-Rust LLM Inference Without a Python Runtime" (hysenlabs.com):
//   section "What actually sits between the request and the tokens" — cached K/V rows are
//   Walsh-Hadamard rotated and absmax-quantized per head; section "TurboQuant is a memory
//   trade, and the README does not price it fully" — attention dequantizes the cache on
//   every step. Paging: infero landing page, section "Beyond plain text decode", item
//   "Continuous batching". Splitting one sequence over several workgroups and merging
//   with log-sum-exp mirrors the flash-attention split count of the infr page ("Introducing
//   infr: A Pure-Rust, Vulkan-First LLM Inference Engine", section "Configuration Without
//   Surprises").
//
// H is orthonormal, so q.k = (Hq).(Hk): the query is rotated once (q' = Hq), scores are taken
// against the stored rotated rows, and the value sum, formed in the rotated space, is rotated
// back at the end (H is its own inverse).
//
// The grouped-query tile is a dense contraction, so both products run on the matrix cores:
//
//   QK  v_mfma_i32_16x16x64_i8. Rows = 16 tokens, columns = the g query heads of the kv head
//       (g <= 16). The rotated query is rounded to an integer q (|q| <= 127 * 2^16, one fp32
//       scale per head, so every element is within 2^-23 of the head's largest) and split into
//       three signed 8-bit digits, q = 65536 d2 + 256 d1 + d0. A K code c enters as the signed
//       byte c * 2^(8 - bits) (the code's bits moved to the top of the byte: two instructions
//       per four codes, no bias), so each digit's integer dot product is exact up to that power
//       of two, folded into the query scale; the three are summed in fp32. Two MFMAs per digit
//       cover 128 dims. (Two digits, q <= 32000, left a query with one dominant rotated element
//       -- a constant offset maps to sqrt(128) e0 -- only 2^-15 of that element on the others,
//       which moved outputs by up to 3e-2 on keys with outlier channels.)
//   PV  v_mfma_f32_16x16x32_f16. Rows = heads, k = 32 tokens, columns = 16 dimensions (eight
//       MFMAs cover 128). The weight of token t for head h is P'[h,t] = p[h,t] * s_v[t], split
//       into an fp16 high part (round toward zero) and the fp16 remainder; each enters its own
//       MFMA, so the weights carry ~22 bits. A V code c enters as an fp16 subnormal whose
//       mantissa holds (c + bias) in the top bits of its low byte, exact, made with one byte
//       permute per pair of tokens. The same weights times the bias alone accumulate in one
//       more tile (two MFMAs against a constant operand) and are subtracted at the end.
//       (Measured on gfx950: with the code in the low mantissa bits instead, the accumulating
//       MFMA loses up to 2^-13 of a code step; in the top bits of the low byte below 2^-18.)
//   bf16 cache: q and K are bf16 operands of v_mfma_f32_16x16x32_bf16 (exact products), the
//       weights are split into bf16 high and low parts against bf16 V.
//   fp8 (E4M3) cache: the bf16 path, with every K and V byte pair widened to two bf16 values by
//       v_cvt_scalef32_pk_bf16_fp8 (unit scale; every E4M3 value, subnormals included, is a bf16
//       normal, so the widening is exact). The fp8 matrix-core instruction (16x16x128, E4M3 K
//       bytes against the query as two E4M3 digits) was tried first: on keys with x30 outlier
//       channels its scores drifted by about 2^-13 of their size, which is more than the 2e-3
//       output tolerance allows.
//
// Online softmax runs in the log2 domain against a per-head reference that moves only when a
// score beats it by more than 2^8. For turbo caches the reference tracks score + e(s_v), e the
// fp16 exponent field of the value scale, so every fp16 weight P' stays below 2^15 whatever
// the scales are, while the normaliser sum(p) is kept in fp32.
//
// Work split: one wave per (split, kv head, row block), walking the split's 32-token tiles in
// order with one softmax state; a tile is two 16-token halves (two pages at page size 16). A
// decode row block is one sequence; a chunked prefill packs 16 / g query tokens of the chunk
// into the 16 columns (one causal limit per column). Scores come out of the QK MFMA exactly
// where the PV MFMA wants its weights (lane l = 16 g + c: head c, tokens 4 g + r), so no data
// moves between the two products. Code bytes are read with buffer loads against a resource
// descriptor (the pool's, or the page block's for pools past 4 GiB; a read past it returns zero)
// and a block-table window held in registers. For turbo4, turbo8 and turbo3 the loads go
// straight to LDS (a ring of DEPTH tile slots per wave, DEPTH picked at launch from how many
// waves share a compute unit): turbo4/turbo8 with lane offsets that leave every operand read
// linear in the lane index and V transposed, turbo3 as the rows are stored. turbo2, bf16 and
// fp8 load into registers, three tiles (two for bf16) in flight. Where sequences have several
// partitions, a wave raises its issue priority in step with the tiles it has left (four levels),
// so that the waves a SIMD runs together finish together instead of in dispatch order.
//
// Each wave prepares the query digits of its kv head's query heads itself (rotation by an
// in-register FWHT, scaling, digit split, packing in the operand layout), from rows fetched by
// LDS DMA ahead of its first tiles.
// A row that fits one split is normalised, rotated back and stored by its wave; otherwise
// (m, l, acc) partials go to the workspace and decode_combine_kernel merges them by
// log-sum-exp, rotates back and stores. An optional host plan (seq_order) only changes which
// slot of the unit order runs which sequence.
#include "row_codec.h"
#include "xq_internal.h"

#include <algorithm>
#include <type_traits>

namespace xq {
namespace {

constexpr int D = kHeadDim;
constexpr int kThreads = 64;              // one wave per work unit
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRotC = 0x1.6a09e6p-4f;   // fp32 nearest to 1/sqrt(128)
constexpr float kLazy = 8.0f;             // rescale only when a score beats m by > 2^8
constexpr int kDigits = 3;                // signed 8-bit digits of the integer query
constexpr float kQiMax = 127.f * 65536.f; // |q| bound: 65536 d2 + 256 d1 + d0, digits in [-128, 127]
constexpr float kWeightExp = 21.f;
// Initial softmax reference: finite, so that a column with no token in its split (a prefill
// query whose position lies before the split) gets weights 2^(-inf - ref) = 0 rather than NaN;
// the first real score always moves the reference (it beats kNoRef by far more than 2^8).
constexpr float kNoRef = -1e30f;        // P' < 2^(w - m + 7): at most 2^15 in fp16
constexpr int kBufferConfig = 0x00020000;   // gfx9 buffer descriptor word 3
// Cache policy of every cache read: non-temporal. Each code byte is read once per decode step,
// so there is nothing to keep; measured on MI355X, random 1 KB page blocks stream at about
// 6.5 TB/s with the bit and 5.5-5.8 TB/s without it.
constexpr int kStream = 2;
// Tiles in flight per wave (register path; bf16 tiles are four times larger).
template <int DT> constexpr int kDepthOf = DT == 0 ? 2 : 3;
// Cache types whose rows are Walsh-Hadamard rotated (the turbo types): the output is rotated
// back. bf16 and fp8 rows are stored unrotated.
template <int DT> constexpr bool kRotated = DT >= 2 && DT <= 8;
// Cache types whose products run on the bf16 matrix-core instructions (unscaled rows).
template <int DT> constexpr bool kBf16Mma = DT == 0 || DT == kFp8;

// LDS staging of code bytes (turbo4, turbo8). Per 16-token half, the K and V code rows of the
// half arrive by DMA (buffer_load_dwordx4 ... lds: 64 lanes x 16 B, lane i written at
// LDS + 16 i) with per-lane source offsets chosen so that every operand read is linear in the
// lane index (no LDS bank conflicts) and V comes out transposed. A slot holds one tile:
// [K half 0][K half 1][V half 0][V half 1][scales: K h0, K h1, V h0, V h1, 32 B each, moved
// by eight lanes of a dword DMA]; each wave owns kDepth slots. With everything staged, the
// loop issues no vector loads into registers, so the only vector-memory waits in it are the
// explicit ones below. kOps is the vector-memory instruction count of one tile (exact: those
// waits count them).
template <int DT> struct Stage {
  static constexpr bool kOn = false;
  static constexpr int kHalf = 0, kDma = 0, kOps = 0, kSlot = 0;
};
// kOps: vector-memory instructions per staged tile with a pool-wide descriptor (the per-page
// descriptor path issues two more; waiting on the smaller count is then merely conservative,
// since loads complete in issue order).
template <> struct Stage<4> {
  static constexpr bool kOn = true;
  static constexpr int kHalf = 1024, kDma = 1, kOps = 4 * kDma + 2, kSlot = 4 * kHalf + 128;
};
template <> struct Stage<8> {
  static constexpr bool kOn = true;
  static constexpr int kHalf = 2048, kDma = 2, kOps = 4 * kDma + 2, kSlot = 4 * kHalf + 128;
};
// turbo3: a half's 16 code rows (768 B, contiguous in the page block) are copied as they are by
// one DMA of 16 B per lane; the last 16 lanes land in the 256 B of padding that follow.
template <> struct Stage<3> {
  static constexpr bool kOn = true;
  static constexpr int kHalf = 1024, kDma = 1, kOps = 4 * kDma + 2, kSlot = 4 * kHalf + 128;
};
// turbo2: the same, a half's 16 rows being 512 B (lanes 32..63 land in the padding).
template <> struct Stage<2> {
  static constexpr bool kOn = true;
  static constexpr int kHalf = 1024, kDma = 1, kOps = 4 * kDma + 2, kSlot = 4 * kHalf + 128;
};
// Layouts that pair (turbo4, turbo8, turbo3, turbo2) or quad (turbo4, turbo8) token blocks in
// the QK tile; the other types use the one-block layout.
template <int DT> constexpr bool kPairOk = DT == 4 || DT == 8 || DT == 3 || DT == 2;
template <int DT> constexpr bool kQuadOk = DT == 4 || DT == 8;
constexpr int kLdsPerCu = 160 * 1024;
// LDS for the wave's query preparation: kMaxGroup raw rows of 256 B land there; the digits of
// up to kQPhaseRows rows (kQRowBytes each, the operand layout) and every row's fp32 score scale
// then take its start. Units with more query columns write and read their digits in two phases.
constexpr int kQRowBytes = 128 * kDigits;
constexpr int kQPhaseRows = 8;
constexpr int kQueryScaleOff = kQPhaseRows * kQRowBytes;
constexpr int kQueryLds = kMaxGroup * 256 > kQueryScaleOff + kMaxGroup * 4 ? kMaxGroup * 256
                                                                            : kQueryScaleOff + kMaxGroup * 4;
static_assert(Stage<4>::kSlot >= kQueryLds && Stage<8>::kSlot >= kQueryLds && Stage<3>::kSlot >= kQueryLds &&
                  Stage<2>::kSlot >= kQueryLds,
              "query rows fit one ring slot");
// Paired-block QK (turbo4, turbo8): with at most this many query heads per kv head, the 16
// columns of the QK tile hold two 16-token blocks of the tile side by side.
constexpr int kPairMaxGroup = 8;
constexpr int kMaxVmcnt = 63;

// Wait until at most N vector-memory instructions of this wave are outstanding. The memory
// clobber keeps the compiler from moving LDS reads of a staged slot above the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for the tile that has `after` tiles (of OPS instructions each) staged behind it.
template <int OPS, int A, int MAXA>
__device__ __forceinline__ void wait_tiles(int after) {
  if constexpr (A == MAXA) {
    wait_vm<A * OPS>();
  } else {
    if (after == A) wait_vm<A * OPS>();
    else wait_tiles<OPS, A + 1, MAXA>(after);
  }
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v3i __attribute__((ext_vector_type(3)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Per cache type: bytes of a code row; the power of two a K code carries in its QK byte
// (c * kKMul); the bias of V codes and the power of two a V operand carries
// ((c + bias) * 2^-kVShift).
template <int DT> struct Codec;
template <> struct Codec<4> { static constexpr int kRow = 64, kKMul = 16, kVBias = 8, kVShift = 20; };
template <> struct Codec<3> { static constexpr int kRow = 48, kKMul = 32, kVBias = 4, kVShift = 19; };
template <> struct Codec<2> { static constexpr int kRow = 32, kKMul = 64, kVBias = 2, kVShift = 18; };
template <> struct Codec<8> { static constexpr int kRow = 128, kKMul = 1, kVBias = 128, kVShift = 24; };
template <> struct Codec<0> { static constexpr int kRow = 256, kKMul = 1, kVBias = 0, kVShift = 0; };
template <> struct Codec<kFp8> { static constexpr int kRow = 128, kKMul = 1, kVBias = 0, kVShift = 0; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Eight 3-bit fields, bytes o .. o + 2 of the eight bytes hi:lo (lo = bytes 0..3), -> two fields
// per byte: field 2i in bits 0..2 and field 2i+1 in bits 3..5 of byte i (bits 6 and 7 are left
// undefined). A shift by 5 (by 2) and the mask 0xe0 then give the even (odd) fields in the top
// three bits of their bytes. sel = spread_sel(o). Four operations: a byte gather (bytes o, o + 1
// to the low half, o + 1, o + 2 to the high half: fields 0..3 at bits 0..11, fields 4..7 at bits
// 20..31), the high half shifted down by 4 on its own (a packed 16-bit shift), and fields 2, 3
// and 6, 7 moved up by 2 into the next byte.
constexpr uint32_t spread_sel(int o) {
  return (uint32_t)o | (uint32_t)(o + 1) << 8 | (uint32_t)(o + 1) << 16 | (uint32_t)(o + 2) << 24;
}
__device__ __forceinline__ uint32_t spread3to6(uint32_t hi, uint32_t lo, uint32_t sel) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t y = __builtin_amdgcn_perm(hi, lo, sel);
  const uint32_t z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, y) >> u16x2{0, 4});
  return (z & 0x003f003fu) | ((z << 2) & ~0x003f003fu);
}

// ---------------------------------------------------------------------------------------
// Query preparation, done by the decode wave itself: q' = H q, q = rint(q' * kQiMax / max|q'|),
// three signed digits, packed in the QK operand layout. The G query rows of the kv head arrive
// in LDS (row h at 256 h, bf16). The whole wave takes part: head h < G owns the aligned group of
// 128 / NPL lanes starting at lane (128 / NPL) h, and lane r of the group holds the NPL
// consecutive dimensions [NPL r, NPL r + NPL) (NPL = 8 for G <= 4, 16 for G <= 8, else 32).
// The FWHT stages below NPL run in-lane, the others exchange with lane r ^ (stage / NPL). Every
// lane has read its raw row before any digit is written (one wave, its LDS operations in
// order). Digit k of dimension d of a row goes to byte 96 (d >> 5) + operand_byte(d & 31) +
// 16 k of the row's kQRowBytes, which other lanes read as operands; the score scale of head h
// goes to sc[h].
// ---------------------------------------------------------------------------------------
// Value held by lane (lane ^ M), M = 1, 2, 4 or 8: DPP quad_perm (M = 1, 2) and row_ror:8
// (M = 8) are VALU operand modifiers; M = 4 is a ds_swizzle in bit-mask mode (no memory access).
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (M == 1 || M == 2) {
    constexpr int kCtrl = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] and [2,3,0,1]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
  } else if constexpr (M == 8) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true));
  } else {
    static_assert(M == 4, "lane exchanges within 16 lanes");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
  }
}

// One cross-lane FWHT stage: the lane whose bit M is clear holds the lower dimension a and gets
// a + b; its partner gets a - b.
template <int M, int N>
__device__ __forceinline__ void fwht_cross(float (&x)[N], int r) {
  const bool upper = (r & M) != 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float other = lane_xor<M>(x[e]);
    x[e] = upper ? other - x[e] : x[e] + other;
  }
}

// Operand byte (digit 0) of dimension e (0..31) of a 32-dimension group: 48 m + 4 w + b for
// operand half/chunk m, dword w, byte b (digits 1 and 2 follow at + 16 and + 32). The map is
// linear in the bits of e.
//   turbo8 (both layouts):              e = 16 m + 4 w + b
//   paired-block turbo4:                e = 16 m + 8 (w >> 1) + 2 b + (w & 1)
//   one-block turbo4/turbo3 (m = chunk): e = 8 w + 2 b + m
//   turbo2 (one-block):                 e = 16 m + 4 b + w
template <int DT, bool PAIRED>
__device__ __forceinline__ int operand_byte(int e) {
  int m, w, b;
  if constexpr (DT == 8) {
    m = e >> 4; w = (e >> 2) & 3; b = e & 3;
  } else if constexpr (DT == 2) {
    m = e >> 4; w = e & 3; b = (e >> 2) & 3;
  } else if constexpr (PAIRED) {
    m = e >> 4; w = 2 * ((e >> 3) & 1) + (e & 1); b = (e >> 1) & 3;
  } else {
    m = e & 1; w = e >> 3; b = (e >> 1) & 3;
  }
  return 16 * kDigits * m + 4 * w + b;
}

// One lane's share of a rotated query row: dimensions [NPL r, NPL r + NPL), the factor that
// maps them to integers (kQiMax / max|q'|, signed like the softmax scale) and the head's score
// scale.
template <int NPL> struct QueryLane {
  float x[NPL];
  float inv;
  float sc;
};

template <int DT, int NPL>
__device__ __forceinline__ void rotate_query_lane(const uint8_t* qa, int h, int r, float softmax_scale,
                                                  QueryLane<NPL>& o) {
  static_assert(NPL == 8 || NPL == 16 || NPL == 32, "8..32 dimensions per lane");
  constexpr int kLanes = 128 / NPL;
  float (&x)[NPL] = o.x;
  const uint4* src = reinterpret_cast<const uint4*>(qa + 256 * h + 2 * NPL * r);
#pragma unroll
  for (int i = 0; i < NPL / 8; ++i) {
    const uint4 w = src[i];
    x[8 * i + 0] = bf16_lo(w.x); x[8 * i + 1] = bf16_hi(w.x);
    x[8 * i + 2] = bf16_lo(w.y); x[8 * i + 3] = bf16_hi(w.y);
    x[8 * i + 4] = bf16_lo(w.z); x[8 * i + 5] = bf16_hi(w.z);
    x[8 * i + 6] = bf16_lo(w.w); x[8 * i + 7] = bf16_hi(w.w);
  }
#pragma unroll
  for (int hh = 1; hh < NPL; hh <<= 1) {
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      if ((e & hh) == 0) {
        const float a = x[e], c = x[e + hh];
        x[e] = a + c;
        x[e + hh] = a - c;
      }
    }
  }
  fwht_cross<1>(x, r);
  fwht_cross<2>(x, r);
  if constexpr (kLanes > 4) fwht_cross<4>(x, r);
  if constexpr (kLanes > 8) fwht_cross<8>(x, r);
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    x[e] *= kRotC;
    am = fmaxf(am, fabsf(x[e]));
  }
  am = fmaxf(am, lane_xor<1>(am));
  am = fmaxf(am, lane_xor<2>(am));
  if constexpr (kLanes > 4) am = fmaxf(am, lane_xor<4>(am));
  if constexpr (kLanes > 8) am = fmaxf(am, lane_xor<8>(am));
  // The score scale is made positive (the sign goes into the digits) and nonzero (a zero
  // query or scale gives zero digits), so a maximum over unscaled scores is the maximum of the
  // scores. A K byte is c * kKMul, so the integer dot product is kKMul times q.c.
  float sc = am > 0.f ? (am / kQiMax) * softmax_scale * kLog2e / (float)Codec<DT>::kKMul : 0.f;
  const bool zero = !(sc != 0.f);
  o.inv = zero ? 0.f : (sc < 0.f ? -kQiMax : kQiMax) / am;
  o.sc = zero ? 1.f : fabsf(sc);
}

// Digits of the lane's dimensions into row `row` of the digit area at qa (and the head's score
// scale into sc_out[h] from lane r = 0).
template <int DT, bool PAIRED, int NPL>
__device__ __forceinline__ void write_query_digits(const QueryLane<NPL>& o, uint8_t* qa, float* sc_out, int h,
                                                   int row, int r) {
  const int d0 = NPL * r;   // the lane's dimensions are d0 + e, e < NPL, with d0 a multiple of NPL
  uint8_t* dst = qa + kQRowBytes * row + 32 * kDigits * (d0 >> 5) + operand_byte<DT, PAIRED>(d0 & 31);
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    // |q| <= kQiMax + 1 (the product rounds once): digits q = 65536 d2 + 256 d1 + d0, each in
    // [-128, 127]
    const int q = (int)rintf(o.x[e] * o.inv);
    const int g0 = ((q + 128) & 255) - 128;
    const int q1 = (q - g0) >> 8;
    const int g1 = ((q1 + 128) & 255) - 128;
    const int g2 = (q1 - g1) >> 8;
    const int off = operand_byte<DT, PAIRED>(e);
    dst[off] = (uint8_t)g0;
    dst[off + 16] = (uint8_t)g1;
    dst[off + 32] = (uint8_t)g2;
  }
  if (r == 0) sc_out[h] = o.sc;
}

// q.c from the three digits' integer dot products: 65536 s2 + 256 s1 + s0. Each |s_k| < 2^21,
// so the low part is exact in int32; the sum is rounded to fp32.
__device__ __forceinline__ float digit_sum(int s0, int s1, int s2) {
  return __builtin_fmaf((float)s2, 65536.f, (float)((s1 << 8) + s0));
}

// ---------------------------------------------------------------------------------------
// Raw bytes of one 32-token tile as one lane holds them.
// ---------------------------------------------------------------------------------------
template <int DT> struct Tile;
template <> struct Tile<4> { v4i k[2]; int v[8]; v2i ks[2], vs[2]; };
template <> struct Tile<3> { v3i k[2]; v2i v[8]; v2i ks[2], vs[2]; };
template <> struct Tile<2> { v2i k[2]; int v[8]; v2i ks[2], vs[2]; };
template <> struct Tile<8> { v4i k[2][2]; v2i v[8]; v2i ks[2], vs[2]; };
template <> struct Tile<0> { v4i k[2][4]; v4i v[8]; };
template <> struct Tile<kFp8> { v4i k[2][2]; v2i v[8]; };

// Wave-uniform view of one 16-token half of a tile: buffer descriptors of the page's K and V
// blocks, the byte offset of the half's first code row and of its first scale.
struct HalfAddr {
  __amdgpu_buffer_rsrc_t k, v;
  int row, scale;
};

// Loop-invariant lane offsets (bytes) from a half's first row (K, V) or first scale.
struct LaneOffsets {
  int k;      // this lane's K bytes: row c, dimension group g
  int v;      // this lane's V bytes of row 4 g (rows 4 g + r follow at r * row bytes)
  int s;      // this lane's four scales (tokens 4 g .. 4 g + 3)
};

template <int DT>
__device__ __forceinline__ LaneOffsets lane_offsets(int col, int g) {
  constexpr int R = Codec<DT>::kRow;
  LaneOffsets o;
  o.k = col * R + g * (R / 4);
  if constexpr (DT == 4) o.v = 4 * g * R + 4 * col;
  else if constexpr (DT == 3) o.v = 4 * g * R + 4 * ((3 * col) >> 2);
  else if constexpr (DT == 2) o.v = 4 * g * R + 4 * (col >> 1);   // dims 16 (c >> 1) .. + 15
  else if constexpr (DT == 8 || DT == kFp8) o.v = 4 * g * R + 8 * col;
  else o.v = 4 * g * R + 16 * col;
  o.s = 8 * g;
  return o;
}

template <int DT>
__device__ __forceinline__ void load_tile(Tile<DT>& t, const HalfAddr (&a)[2], const LaneOffsets& o) {
  constexpr int R = Codec<DT>::kRow;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (DT == 4) {
      t.k[h] = __builtin_amdgcn_raw_buffer_load_b128(a[h].k, o.k, a[h].row, kStream);
    } else if constexpr (DT == 3) {
      t.k[h] = __builtin_amdgcn_raw_buffer_load_b96(a[h].k, o.k, a[h].row, kStream);
    } else if constexpr (DT == 2) {
      t.k[h] = __builtin_amdgcn_raw_buffer_load_b64(a[h].k, o.k, a[h].row, kStream);
    } else if constexpr (DT == 8 || DT == kFp8) {
      t.k[h][0] = __builtin_amdgcn_raw_buffer_load_b128(a[h].k, o.k, a[h].row, kStream);
      t.k[h][1] = __builtin_amdgcn_raw_buffer_load_b128(a[h].k, o.k + 16, a[h].row, kStream);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        t.k[h][i] = __builtin_amdgcn_raw_buffer_load_b128(a[h].k, o.k + 16 * i, a[h].row, kStream);
    }
    if constexpr (has_scales(DT)) {
      t.ks[h] = __builtin_amdgcn_raw_buffer_load_b64(a[h].k, o.s, a[h].scale, kStream);
      t.vs[h] = __builtin_amdgcn_raw_buffer_load_b64(a[h].v, o.s, a[h].scale, kStream);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * h + r;
      if constexpr (DT == 4 || DT == 2) {
        t.v[j] = __builtin_amdgcn_raw_buffer_load_b32(a[h].v, o.v + r * R, a[h].row, kStream);
      } else if constexpr (DT == 3 || DT == 8 || DT == kFp8) {
        // turbo3: dims 8c..8c+7 are bits [24c, 24c+24) of the row; the second dword of the
        // last group lies in the next row or the block's scale area, both inside the block
        t.v[j] = __builtin_amdgcn_raw_buffer_load_b64(a[h].v, o.v + r * R, a[h].row, kStream);
      } else {
        t.v[j] = __builtin_amdgcn_raw_buffer_load_b128(a[h].v, o.v + r * R, a[h].row, kStream);
      }
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// Per-lane source offsets of the staging DMAs (bytes from a half's first row).
struct DmaOffsets {
  int k[2];   // K chunk m: row c = i % 16, bytes of dimension group g = i / 16
  int v[2];   // V chunk m: rows 4 g + r, the 16 bytes each lane of a row group needs
};

template <int DT>
__device__ __forceinline__ DmaOffsets dma_offsets(int lane) {
  DmaOffsets o{};
  if constexpr (DT == 4) {
    o.k[0] = (lane & 15) * 64 + 16 * (lane >> 4);
    o.v[0] = (4 * ((lane >> 2) & 3) + (lane >> 4)) * 64 + 16 * (lane & 3);
  } else if constexpr (DT == 3 || DT == 2) {
    o.k[0] = 16 * lane;   // as stored: row c of the half at 48 c (turbo2: 32 c)
    o.v[0] = 16 * lane;
  } else if constexpr (DT == 8) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      o.k[m] = (lane & 15) * 128 + 32 * (lane >> 4) + 16 * m;
      o.v[m] = (4 * ((lane >> 3) & 3) + 2 * m + (lane >> 5)) * 128 + 16 * (lane & 7);
    }
  }
  return o;
}

// Issue the staging DMAs of one tile into `slot`.
template <int DT, bool FLAT>
__device__ __forceinline__ void stage_tile(uint8_t* slot, const HalfAddr (&a)[2], const DmaOffsets& d,
                                           int lane) {
  using S = Stage<DT>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int m = 0; m < S::kDma; ++m) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a[h].k, (lds_void*)(slot + h * S::kHalf + 1024 * m), 16,
                                               d.k[m], a[h].row, 0, kStream);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a[h].v, (lds_void*)(slot + (2 + h) * S::kHalf + 1024 * m), 16,
                                               d.v[m], a[h].row, 0, kStream);
    }
  }
  // the 16 scales of each half: eight lanes per half, one dword each. With one descriptor for
  // the whole pool both halves go in one instruction (lanes 0..7: half 0, 8..15: half 1).
  if constexpr (FLAT) {
    if (lane < 16) {
      const int off = (lane < 8 ? a[0].scale : a[1].scale) + 4 * (lane & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a[0].k, (lds_void*)(slot + 4 * S::kHalf), 4, off, 0, 0, kStream);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a[0].v, (lds_void*)(slot + 4 * S::kHalf + 64), 4, off, 0, 0, kStream);
    }
  } else if (lane < 8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a[h].k, (lds_void*)(slot + 4 * S::kHalf + 32 * h), 4, 4 * lane,
                                               a[h].scale, 0, kStream);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a[h].v, (lds_void*)(slot + 4 * S::kHalf + 64 + 32 * h), 4,
                                               4 * lane, a[h].scale, 0, kStream);
    }
  }
}

// Issue priority of a unit's wave when sequences have several partitions (units of about equal
// length): a SIMD's arbiter favours its oldest wave, so of the units sharing a SIMD the ones
// dispatched later fall behind and end the call. Each step the wave takes a priority from the
// tiles it has left, in four levels of kPrioTiles tiles, so that the waves with the most work
// left issue first.
constexpr int kPrioTiles = 8;
__device__ __forceinline__ void issue_priority(int tiles_left) {
  if (tiles_left > 3 * kPrioTiles) __builtin_amdgcn_s_setprio(3);
  else if (tiles_left > 2 * kPrioTiles) __builtin_amdgcn_s_setprio(2);
  else if (tiles_left > kPrioTiles) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Operand bytes of a staged tile, read from its slot.
template <int DT>
__device__ __forceinline__ void read_slot(Tile<DT>& t, const uint8_t* slot, int lane) {
  using S = Stage<DT>;
  const int g = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    t.ks[h] = *reinterpret_cast<const v2i*>(slot + 4 * S::kHalf + 32 * h + 8 * g);
    t.vs[h] = *reinterpret_cast<const v2i*>(slot + 4 * S::kHalf + 64 + 32 * h + 8 * g);
    if constexpr (DT == 2) {
      // the bytes the register path loads: K row c, bytes 8 g .. 8 g + 7; V rows 4 g + r, the
      // dword of dims 16 (c >> 1) .. + 15
      const int col = lane & 15;
      const int* kr = reinterpret_cast<const int*>(slot + h * S::kHalf + 32 * col + 8 * g);
      t.k[h] = v2i{kr[0], kr[1]};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        t.v[4 * h + r] = *reinterpret_cast<const int*>(slot + (2 + h) * S::kHalf + 32 * (4 * g + r) + 4 * (col >> 1));
    } else if constexpr (DT == 3) {
      // the bytes the register path loads: K row c, bytes 12 g .. 12 g + 11; V rows 4 g + r, the
      // two dwords from byte 4 ((3 c) >> 2) (read as dwords: the offsets are 4-byte aligned)
      const int col = lane & 15;
      const int* kr = reinterpret_cast<const int*>(slot + h * S::kHalf + 48 * col + 12 * g);
      t.k[h] = v3i{kr[0], kr[1], kr[2]};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int* vr = reinterpret_cast<const int*>(slot + (2 + h) * S::kHalf + 48 * (4 * g + r) + 4 * ((3 * col) >> 2));
        t.v[4 * h + r] = v2i{vr[0], vr[1]};
      }
    } else if constexpr (DT == 4) {
      t.k[h] = *reinterpret_cast<const v4i*>(slot + h * S::kHalf + 16 * lane);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        t.v[4 * h + r] = *reinterpret_cast<const int*>(slot + (2 + h) * S::kHalf + 256 * r + 4 * lane);
    } else if constexpr (DT == 8) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
        t.k[h][m] = *reinterpret_cast<const v4i*>(slot + h * S::kHalf + 1024 * m + 16 * lane);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        t.v[4 * h + r] = *reinterpret_cast<const v2i*>(slot + (2 + h) * S::kHalf + 512 * r + 8 * lane);
    }
  }
}

// K codes of one half as QK operand bytes c * kKMul, for the two k-chunks of the MFMA.
template <int DT>
__device__ __forceinline__ void k_operands(const Tile<DT>& t, int h, v4i& a0, v4i& a1) {
  if constexpr (DT == 4) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = (uint32_t)t.k[h][w];
      a0[w] = (int)((x << 4) & 0xf0f0f0f0u);        // dims 32g + 8w + 2b: 16 c
      a1[w] = (int)(x & 0xf0f0f0f0u);               // dims 32g + 8w + 2b + 1: 16 c
    }
  } else if constexpr (DT == 3) {
    const uint32_t d0 = (uint32_t)t.k[h][0], d1 = (uint32_t)t.k[h][1], d2 = (uint32_t)t.k[h][2];
    // fields 8 w .. 8 w + 7: bytes 3 w .. 3 w + 2 of d0 d1 d2
    const uint32_t grp[4] = {spread3to6(d1, d0, spread_sel(0)), spread3to6(d1, d0, spread_sel(3)),
                             spread3to6(d2, d1, spread_sel(2)), spread3to6(d2, d1, spread_sel(5))};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t n = grp[w];                           // raw 3-bit fields, two per byte
      a0[w] = (int)((n << 5) & 0xe0e0e0e0u);               // 32 c
      a1[w] = (int)((n << 2) & 0xe0e0e0e0u);
    }
  } else if constexpr (DT == 2) {
    // dword i holds dims 16 i .. 16 i + 15 of the lane's 32, code 4 b + w in bits 2 w of byte b;
    // shifting field w to the top of each byte gives 64 c: chunk m, dword w, byte b is dim
    // 16 m + 4 b + w
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      a0[w] = (int)(((uint32_t)t.k[h][0] << (6 - 2 * w)) & 0xc0c0c0c0u);
      a1[w] = (int)(((uint32_t)t.k[h][1] << (6 - 2 * w)) & 0xc0c0c0c0u);
    }
  } else {  // turbo8: signed bytes as stored
    a0 = t.k[h][0];
    a1 = t.k[h][1];
  }
}

// V codes of the eight token slots as bytes whose top bits hold (code + bias): byte i of e[j]
// is dimension 8 c + 2 i (turbo8: 8 c + i), of o[j] dimension 8 c + 2 i + 1 (turbo8: 8 c + 4 + i).
// Paired with a zero byte, such a byte is an fp16 subnormal, exactly (code + bias) * 2^-kVShift.
template <int DT>
__device__ __forceinline__ void v_bytes(const Tile<DT>& t, uint32_t (&e)[8], uint32_t (&o)[8], int col) {
  if constexpr (DT == 4) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = (uint32_t)t.v[j] ^ 0x88888888u;   // c + 8 per nibble
      e[j] = (u << 4) & 0xf0f0f0f0u;                       // even dims, (c + 8) << 4
      o[j] = u & 0xf0f0f0f0u;                              // odd dims, already in the high nibble
    }
  } else if constexpr (DT == 3) {
    // the lane's 8 dims start at byte (3 col) mod 4 of its two dwords
    const uint32_t sel = spread_sel((3 * col) & 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // two fields per byte, the top bit of each flipped: c + 4
      const uint32_t n = spread3to6((uint32_t)t.v[j][1], (uint32_t)t.v[j][0], sel) ^ 0x24242424u;
      e[j] = (n << 5) & 0xe0e0e0e0u;                       // (c + 4) << 5
      o[j] = (n << 2) & 0xe0e0e0e0u;
    }
  } else if constexpr (DT == 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e[j] = (uint32_t)t.v[j][0] ^ 0x80808080u;     // c + 128
      o[j] = (uint32_t)t.v[j][1] ^ 0x80808080u;
    }

  } else if constexpr (DT == 2) {
    // the lane's 8 dims are the low or high 16 bits of the loaded dword; their bytes go to
    // bytes 0 and 2, then nibble i (dims 8 c + 2 i, 8 c + 2 i + 1) to byte i
    const uint32_t sel = (col & 1) ? 0x0c030c02u : 0x0c010c00u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = perm(0u, (uint32_t)t.v[j] ^ 0xaaaaaaaau, sel);   // c + 2 per field
      const uint32_t n = (u & 0x000f000fu) | ((u << 4) & 0x0f000f00u);
      e[j] = (n << 6) & 0xc0c0c0c0u;                // (c + 2) << 6
      o[j] = (n << 4) & 0xc0c0c0c0u;
    }
  }
}

// bf16 matrix-core operands. K: the 8 dimensions 32 g + 8 m .. + 7 of the lane's token; V: dword i
// (dimensions 8 c + 2 i, 8 c + 2 i + 1) of token slot j. fp8 bytes are widened exactly.
template <int DT>
__device__ __forceinline__ v8bf bf16_k_operand(const Tile<DT>& t, int h, int m) {
  if constexpr (DT == kFp8) {
    const v4i& x = t.k[h][m >> 1];
    const int w = 2 * (m & 1);
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)x[w], 1.f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)x[w], 1.f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)x[w + 1], 1.f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)x[w + 1], 1.f, true);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    return __builtin_bit_cast(v8bf, t.k[h][m]);
  }
}
template <int DT>
__device__ __forceinline__ uint32_t bf16_v_dword(const Tile<DT>& t, int j, int i) {
  if constexpr (DT == kFp8) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const uint32_t x = (uint32_t)t.v[j][i >> 1];
    return __builtin_bit_cast(uint32_t, (i & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.f, true)
                                                : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.f, false));
  } else {
    return (uint32_t)t.v[j][i];
  }
}

struct WaveState {
  v4f acc[8];          // PV accumulators: lane (g, c) reg r = head 4g + r, dimension 8c + tau
  v4f accb;            // the same weights times the bias alone (every column equal)
  float m;             // reference of head c (log2 domain)
  float l;             // partial sum of p over this lane's tokens
};

// One 32-token tile: QK, online softmax, PV. When `full` is false (the last tile of a split),
// token slots 16 h + r >= lim are masked.
template <int DT>
__device__ __forceinline__ void process_tile(const Tile<DT>& t, WaveState& st,
                                             const v4i (&qi)[2][kDigits], const v8bf (&qb)[4],
                                             float qs, int lim, int lim_rows, bool full, int col, int g) {
  // ---- scores: y = log2-domain score; w = y + exponent field of s_v (turbo) --------------------
  float y[8], w[8];
  uint32_t sv[8];   // fp16 value scale in the low half (1.0 for bf16)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (!kBf16Mma<DT>) {
      v4i a0, a1;
      k_operands<DT>(t, h, a0, a1);
      const v4i z = {0, 0, 0, 0};
      v4i s[kDigits];
#pragma unroll
      for (int k = 0; k < kDigits; ++k) {
        s[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, qi[0][k], z, 0, 0, 0);
        s[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, qi[1][k], s[k], 0, 0, 0);
      }
      const uint32_t ks[4] = {(uint32_t)t.ks[h][0], (uint32_t)t.ks[h][0] >> 16, (uint32_t)t.ks[h][1],
                              (uint32_t)t.ks[h][1] >> 16};
      const uint32_t vs[4] = {(uint32_t)t.vs[h][0], (uint32_t)t.vs[h][0] >> 16, (uint32_t)t.vs[h][1],
                              (uint32_t)t.vs[h][1] >> 16};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float zf = digit_sum(s[0][r], s[1][r], s[2][r]);
        // fma with a zero addend keeps the fp16 operand in a mixed-precision fma
        y[4 * h + r] = __builtin_fmaf(half_lo(ks[r]), zf * qs, 0.f);
        sv[4 * h + r] = vs[r];
        w[4 * h + r] = y[4 * h + r] + (float)((vs[r] >> 10) & 31u);
      }
    } else {
      v4f s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16_k_operand<DT>(t, h, m), qb[m], s, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[4 * h + r] = s[r] * qs;
        w[4 * h + r] = y[4 * h + r];
        sv[4 * h + r] = 0x3c00u;
      }
    }
  }
  if (!full) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = 16 * (j >> 2) + (j & 3) < lim;
      y[j] = ok ? y[j] : -INFINITY;
      w[j] = ok ? w[j] : -INFINITY;
      sv[j] = ok ? sv[j] : 0u;    // unwritten slots may hold NaN patterns
    }
  }

  // ---- lazily moved reference: each lane tests its own scores; only when some lane of the
  // wave is past the threshold is the head maximum taken across the four lanes of a head ----
  float mx = fmaxf(fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3])), fmaxf(fmaxf(w[4], w[5]), fmaxf(w[6], w[7])));
  if (__builtin_expect(__any(mx > st.m + kLazy), 0)) {
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool up = mx > st.m + kLazy;
    const float f = up ? __builtin_amdgcn_exp2f(st.m - mx) : 1.f;
    st.m = up ? mx : st.m;
    st.l *= f;
    float fr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) fr[r] = __shfl(f, 4 * g + r);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int tau = 0; tau < 8; ++tau) st.acc[tau][r] *= fr[r];
      st.accb[r] *= fr[r];
    }
  }

  // ---- weights: p = 2^(y - m + 21) for the normaliser, P' = p * s_v for the MFMA ---------------
  const float mref = !kBf16Mma<DT> ? st.m - kWeightExp : st.m;
  float pw[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __builtin_amdgcn_exp2f(y[j] - mref);
    st.l += p;
    pw[j] = __builtin_fmaf(half_lo(sv[j]), p, 0.f);
  }
  uint32_t ahi[4], alo[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (!kBf16Mma<DT>) {
      const auto hi2 = __builtin_amdgcn_cvt_pkrtz(pw[2 * k], pw[2 * k + 1]);
      const auto lo2 = __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf((float)hi2[0], -1.f, pw[2 * k]),
                                                  __builtin_fmaf((float)hi2[1], -1.f, pw[2 * k + 1]));
      ahi[k] = __builtin_bit_cast(uint32_t, hi2);
      alo[k] = __builtin_bit_cast(uint32_t, lo2);
    } else {
      const uint32_t b0 = __float_as_uint(pw[2 * k]), b1 = __float_as_uint(pw[2 * k + 1]);
      const float r0 = pw[2 * k] - __uint_as_float(b0 & 0xffff0000u);
      const float r1 = pw[2 * k + 1] - __uint_as_float(b1 & 0xffff0000u);
      ahi[k] = perm(b1, b0, 0x07060302u);
      alo[k] = perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
    }
  }

  // ---- PV -----------------------------------------------------------------------------------
  if constexpr (!kBf16Mma<DT>) {
    const v8h Ahi = __builtin_bit_cast(v8h, make_uint4(ahi[0], ahi[1], ahi[2], ahi[3]));
    const v8h Alo = __builtin_bit_cast(v8h, make_uint4(alo[0], alo[1], alo[2], alo[3]));
    // the bias alone, (bias << (8 - bits)) in every slot: the byte 0x80 for all three types
    if constexpr (Codec<DT>::kVBias != 0) {
      const v8h Bb = __builtin_bit_cast(v8h, make_uint4(0x00800080u, 0x00800080u, 0x00800080u, 0x00800080u));
      st.accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bb, st.accb, 0, 0, 0);
      st.accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bb, st.accb, 0, 0, 0);
    }
    uint32_t e[8], o[8];
    v_bytes<DT>(t, e, o, col);
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      const uint32_t* src;
      int i;
      if constexpr (DT == 8) {
        src = tau < 4 ? e : o;
        i = tau & 3;
      } else {
        src = (tau & 1) ? o : e;
        i = tau >> 1;
      }
      const uint32_t sel = (uint32_t)i | (0x0cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0cu << 24);
      const v8h B = __builtin_bit_cast(v8h, make_uint4(perm(src[1], src[0], sel), perm(src[3], src[2], sel),
                                                       perm(src[5], src[4], sel), perm(src[7], src[6], sel)));
      st.acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, B, st.acc[tau], 0, 0, 0);
      st.acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, B, st.acc[tau], 0, 0, 0);
    }
  } else {
    const v8bf Ahi = __builtin_bit_cast(v8bf, make_uint4(ahi[0], ahi[1], ahi[2], ahi[3]));
    const v8bf Alo = __builtin_bit_cast(v8bf, make_uint4(alo[0], alo[1], alo[2], alo[3]));
    uint32_t vv[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = full || (16 * (j >> 2) + (j & 3) < lim_rows);   // unwritten slots may be NaN
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[j][i] = ok ? bf16_v_dword<DT>(t, j, i) : 0u;
    }
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      const int i = tau >> 1;
      const uint32_t sel = (tau & 1) ? 0x07060302u : 0x05040100u;
      const v8bf B = __builtin_bit_cast(v8bf, make_uint4(perm(vv[1][i], vv[0][i], sel), perm(vv[3][i], vv[2][i], sel),
                                                         perm(vv[5][i], vv[4][i], sel), perm(vv[7][i], vv[6][i], sel)));
      st.acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ahi, B, st.acc[tau], 0, 0, 0);
      st.acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Alo, B, st.acc[tau], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Paired-block tile (turbo4 and turbo8 with G <= 8 query heads per kv head).
//
// The QK tile has 16 columns but a kv head has only G query heads, so column n = G j + h
// (j = 0, 1; n >= 2 G repeats column n mod 2 G) holds head h against token block j (the 16
// tokens of half j of the tile). The query operand is block diagonal over the four k-groups of
// lanes: lane group gg (lanes 16 gg .. 16 gg + 15) carries block gg >> 1, so a column sees its
// own block's keys only. The K operand of lane (gg, t) is token t of block gg >> 1,
// dimensions 32 m + 16 (gg & 1) + [0, 16) in MFMA m (m = 0..3): four MFMAs per digit cover
// 128 dimensions of both blocks, as many as one block takes in the one-block layout. Lane
// (gg, n) then holds the scores of tokens 4 gg + r of block j(n) for head h(n): four values
// where the one-block layout has eight, so the softmax work per tile halves. For PV the same
// values go to k slots r (block 0) or 4 + r (block 1) of the A operand, zeros in the other
// four, matching the V operand of the one-block layout; rows n and G + n of the product are
// the two blocks' partial sums for head n and are added at the end of the unit.
// ---------------------------------------------------------------------------------------
template <int DT> struct PairTile;
template <> struct PairTile<4> {
  v2i k[4];            // raw K code bytes: 8 bytes (16 dims) per MFMA
  int v[8];            // V as in Tile<4>
  v2i ks, vs;          // fp16 scales of tokens 4 gg + r of block j(n)
};
template <> struct PairTile<8> {
  v4i k[4];            // raw K code bytes: 16 bytes (16 dims) per MFMA
  v2i v[8];
  v2i ks, vs;
};
template <> struct PairTile<3> {
  v2i k[4];            // two dwords holding the 48 bits (16 codes) of the lane's 16 dims per MFMA
  v2i v[8];            // V as in Tile<3>
  v2i ks, vs;
};
template <> struct PairTile<2> {
  int k[4];            // the 32 bits (16 codes) of the lane's 16 dims per MFMA
  int v[8];            // V as in Tile<2>
  v2i ks, vs;
};

// Lane roles of the paired layout.
struct PairLane {
  int jn;      // token block of this lane's column (0, 1)
  int hn;      // query head of this lane's column (0 .. G-1)
  int kb;      // token block of this lane's K operand (lane group >> 1)
  int kp;      // which 16 of each 32 dimensions this lane's K operand holds (lane group & 1)
  uint32_t ksel0, ksel1;   // turbo3: byte gathers of its K fields 0..7 and 8..15 (spread3to6)
  uint32_t vsel;           // turbo3: byte gather of its 8 V dims (spread3to6)
};

__device__ __forceinline__ PairLane pair_lane(int lane, int G) {
  const int n = lane & 15, gg = lane >> 4;
  const int ne = n < 2 * G ? n : n % (2 * G);
  const int kp = gg & 1;
  return PairLane{ne / G, ne % G, gg >> 1, kp, spread_sel(2 * kp), spread_sel(2 * kp + 3), spread_sel((3 * n) & 3)};
}

template <int DT>
__device__ __forceinline__ void read_slot_pair(PairTile<DT>& t, const uint8_t* slot, int lane, const PairLane& pl) {
  using S = Stage<DT>;
  const int gg = lane >> 4, tk = lane & 15;
  // scales of tokens 4 gg + r of block jn
  t.ks = *reinterpret_cast<const v2i*>(slot + 4 * S::kHalf + 32 * pl.jn + 8 * gg);
  t.vs = *reinterpret_cast<const v2i*>(slot + 4 * S::kHalf + 64 + 32 * pl.jn + 8 * gg);
  const uint8_t* kh = slot + pl.kb * S::kHalf;
  if constexpr (DT == 2) {
    // rows as stored (32 B): dims 32 m + 16 kp .. + 15 are the dword at byte 8 m + 4 kp
#pragma unroll
    for (int m = 0; m < 4; ++m) t.k[m] = *reinterpret_cast<const int*>(kh + 32 * tk + 8 * m + 4 * pl.kp);
  } else if constexpr (DT == 3) {
    // rows as stored (48 B): dims 32 m + 16 kp .. + 15 are bits 96 m + 48 kp .. + 47 of the row,
    // i.e. bytes 12 m + 6 kp .. + 5: bytes 2 kp .. 2 kp + 5 of the two aligned dwords from byte
    // 12 m + 4 kp (pair_k_operand gathers them)
    const int* kr = reinterpret_cast<const int*>(kh + 48 * tk);
#pragma unroll
    for (int m = 0; m < 4; ++m) t.k[m] = v2i{kr[3 * m + pl.kp], kr[3 * m + pl.kp + 1]};
  } else if constexpr (DT == 4) {
    // half layout: row t, 16-byte chunk c (32 dims) at 16 (t + 16 c)
#pragma unroll
    for (int m = 0; m < 4; ++m) t.k[m] = *reinterpret_cast<const v2i*>(kh + 16 * (tk + 16 * m) + 8 * pl.kp);
  } else {
    // half layout: row t, bytes 32 c + 16 q at 1024 q + 16 (t + 16 c)
#pragma unroll
    for (int m = 0; m < 4; ++m) t.k[m] = *reinterpret_cast<const v4i*>(kh + 1024 * pl.kp + 16 * (tk + 16 * m));
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (DT == 2) {
        t.v[4 * h + r] = *reinterpret_cast<const int*>(slot + (2 + h) * S::kHalf + 32 * (4 * gg + r) + 4 * (tk >> 1));
      } else if constexpr (DT == 3) {
        const int* vr = reinterpret_cast<const int*>(slot + (2 + h) * S::kHalf + 48 * (4 * gg + r) +
                                                     4 * ((3 * tk) >> 2));
        t.v[4 * h + r] = v2i{vr[0], vr[1]};
      } else if constexpr (DT == 4) {
        t.v[4 * h + r] = *reinterpret_cast<const int*>(slot + (2 + h) * S::kHalf + 256 * r + 4 * lane);
      } else {
        t.v[4 * h + r] = *reinterpret_cast<const v2i*>(slot + (2 + h) * S::kHalf + 512 * r + 8 * lane);
      }
    }
  }
}

// K operand of MFMA m: 16 codes as bytes c * kKMul; byte 4 w + b is dimension
// 8 (w >> 1) + 2 b + (w & 1) (turbo4) or 4 w + b (turbo8) of the lane's 16.
template <int DT>
__device__ __forceinline__ v4i pair_k_operand(const PairTile<DT>& t, int m, const PairLane& pl) {
  if constexpr (DT == 2) {
    // code of dim 4 b + w (of the lane's 16) to the top two bits of byte b of dword w: 64 c
    const uint32_t x = (uint32_t)t.k[m];
    return v4i{(int)((x << 6) & 0xc0c0c0c0u), (int)((x << 4) & 0xc0c0c0c0u), (int)((x << 2) & 0xc0c0c0c0u),
               (int)(x & 0xc0c0c0c0u)};
  } else if constexpr (DT == 3) {
    // dims 0..7 and 8..15 of the lane's 16: bytes o .. o + 2 and o + 3 .. o + 5 of the two
    // dwords, o = 2 kp; 32 c in the top of each byte
    const uint32_t k0 = (uint32_t)t.k[m][0], k1 = (uint32_t)t.k[m][1];
    const uint32_t y0 = spread3to6(k1, k0, pl.ksel0);
    const uint32_t y1 = spread3to6(k1, k0, pl.ksel1);
    return v4i{(int)((y0 << 5) & 0xe0e0e0e0u), (int)((y0 << 2) & 0xe0e0e0e0u), (int)((y1 << 5) & 0xe0e0e0e0u),
               (int)((y1 << 2) & 0xe0e0e0e0u)};
  } else if constexpr (DT == 4) {
    const uint32_t x0 = (uint32_t)t.k[m][0], x1 = (uint32_t)t.k[m][1];
    return v4i{(int)((x0 << 4) & 0xf0f0f0f0u), (int)(x0 & 0xf0f0f0f0u), (int)((x1 << 4) & 0xf0f0f0f0u),
               (int)(x1 & 0xf0f0f0f0u)};
  } else {
    return t.k[m];
  }
}

// refill(): called once the tile's products are issued (the ring's next load goes out while
// the matrix cores work).
template <int DT, typename Refill>
__device__ __forceinline__ void process_pair_tile(const PairTile<DT>& t, WaveState& st, const v4i (&qj)[4][kDigits],
                                                  float qs, int lim, bool full, const PairLane& pl, int G,
                                                  int lane, Refill&& refill) {
  // ---- scores: y' = s_k * (q.c) in integer-digit units; the log2-domain score is y' * qs ------
  v4i s[kDigits];
#pragma unroll
  for (int k = 0; k < kDigits; ++k) s[k] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const v4i a = pair_k_operand<DT>(t, m, pl);
#pragma unroll
    for (int k = 0; k < kDigits; ++k) s[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qj[m][k], s[k], 0, 0, 0);
  }
  refill();
  const uint32_t ks[4] = {(uint32_t)t.ks[0], (uint32_t)t.ks[0] >> 16, (uint32_t)t.ks[1], (uint32_t)t.ks[1] >> 16};
  uint32_t sv[4] = {(uint32_t)t.vs[0] & 0xffffu, (uint32_t)t.vs[0] >> 16, (uint32_t)t.vs[1] & 0xffffu,
                    (uint32_t)t.vs[1] >> 16};
  float y[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    y[r] = __builtin_fmaf(half_lo(ks[r]), digit_sum(s[0][r], s[1][r], s[2][r]), 0.f);
  }
  if (!full) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = 16 * pl.jn + r < lim;
      y[r] = ok ? y[r] : -INFINITY;
      sv[r] = ok ? sv[r] : 0u;    // unwritten slots may hold NaN patterns
    }
  }
  // lane bound of w = y + e(s_v): the largest score plus the largest exponent field of the
  // lane's value scales (raw fp16 bits of positive scales order like their values)
  const uint32_t smax = max(max(sv[0], sv[1]), max(sv[2], sv[3]));
  const float ymax = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
  float mx = __builtin_fmaf(ymax, qs, (float)(smax >> 10));
  if (__builtin_expect(__any(mx > st.m + kLazy), 0)) {
    // head maximum over the lanes of head hn: columns hn and G + hn, all four lane groups
    const int pn = pl.jn ? pl.hn : pl.hn + G;
    mx = fmaxf(mx, __shfl(mx, (lane & 48) | pn));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool up = mx > st.m + kLazy;
    const float f = up ? __builtin_amdgcn_exp2f(st.m - mx) : 1.f;
    st.m = up ? mx : st.m;
    st.l *= f;
    // PV row 4 gg + r is column n = 4 gg + r: head (n mod 2G) mod G, whose factor lane n has
    // (computed here from an opaque copy of the lane id, not hoisted into registers the tile
    // loop lacks)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int g4 = (ln >> 4) * 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nr = g4 + r;
      const int ner = nr < 2 * G ? nr : nr % (2 * G);
      const float fr = __shfl(f, ner % G);
#pragma unroll
      for (int tau = 0; tau < 8; ++tau) st.acc[tau][r] *= fr;
      st.accb[r] *= fr;
    }
  }

  // ---- weights: p = 2^(y - m + 21), P' = p * s_v --------------------------------------------
  const float nref = kWeightExp - st.m;
  float pw[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(y[r], qs, nref));
    st.l += pr;
    pw[r] = __builtin_fmaf(half_lo(sv[r]), pr, 0.f);
  }
  const auto h01 = __builtin_amdgcn_cvt_pkrtz(pw[0], pw[1]);
  const auto h23 = __builtin_amdgcn_cvt_pkrtz(pw[2], pw[3]);
  const auto l01 = __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf((float)h01[0], -1.f, pw[0]),
                                              __builtin_fmaf((float)h01[1], -1.f, pw[1]));
  const auto l23 = __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf((float)h23[0], -1.f, pw[2]),
                                              __builtin_fmaf((float)h23[1], -1.f, pw[3]));
  const uint32_t hi01 = __builtin_bit_cast(uint32_t, h01), hi23 = __builtin_bit_cast(uint32_t, h23);
  const uint32_t lo01 = __builtin_bit_cast(uint32_t, l01), lo23 = __builtin_bit_cast(uint32_t, l23);
  const bool b1 = pl.jn != 0;
  const v8h Ahi = __builtin_bit_cast(v8h, make_uint4(b1 ? 0u : hi01, b1 ? 0u : hi23, b1 ? hi01 : 0u, b1 ? hi23 : 0u));
  const v8h Alo = __builtin_bit_cast(v8h, make_uint4(b1 ? 0u : lo01, b1 ? 0u : lo23, b1 ? lo01 : 0u, b1 ? lo23 : 0u));

  // ---- PV (as the one-block layout) -----------------------------------------------------------
  const v8h Bb = __builtin_bit_cast(v8h, make_uint4(0x00800080u, 0x00800080u, 0x00800080u, 0x00800080u));
  st.accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bb, st.accb, 0, 0, 0);
  st.accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bb, st.accb, 0, 0, 0);
  uint32_t e[8], o[8];
  if constexpr (DT == 2) {
    // as v_bytes<2>: the lane's 8 dims are the low or high 16 bits of the dword
    const uint32_t sel = (lane & 1) ? 0x0c030c02u : 0x0c010c00u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = perm(0u, (uint32_t)t.v[j] ^ 0xaaaaaaaau, sel);   // c + 2 per field
      const uint32_t n = (u & 0x000f000fu) | ((u << 4) & 0x0f000f00u);
      e[j] = (n << 6) & 0xc0c0c0c0u;                // (c + 2) << 6
      o[j] = (n << 4) & 0xc0c0c0c0u;
    }
  } else if constexpr (DT == 3) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t n = spread3to6((uint32_t)t.v[j][1], (uint32_t)t.v[j][0], pl.vsel);   // two fields per byte
      e[j] = ((n << 5) & 0xe0e0e0e0u) ^ 0x80808080u;       // (c + 4) << 5: the top bit flipped
      o[j] = ((n << 2) & 0xe0e0e0e0u) ^ 0x80808080u;
    }
  } else if constexpr (DT == 4) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t x = (uint32_t)t.v[j];
      e[j] = ((x << 4) & 0xf0f0f0f0u) ^ 0x80808080u;   // even dims, (c + 8) << 4
      o[j] = (x & 0xf0f0f0f0u) ^ 0x80808080u;          // odd dims
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e[j] = (uint32_t)t.v[j][0] ^ 0x80808080u;     // c + 128
      o[j] = (uint32_t)t.v[j][1] ^ 0x80808080u;
    }
  }
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) {
    const uint32_t* src;
    int i;
    if constexpr (DT == 8) {
      src = tau < 4 ? e : o;
      i = tau & 3;
    } else {
      src = (tau & 1) ? o : e;
      i = tau >> 1;
    }
    const uint32_t sel = (uint32_t)i | (0x0cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0cu << 24);
    const v8h B = __builtin_bit_cast(v8h, make_uint4(perm(src[1], src[0], sel), perm(src[3], src[2], sel),
                                                     perm(src[5], src[4], sel), perm(src[7], src[6], sel)));
    st.acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, B, st.acc[tau], 0, 0, 0);
    st.acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, B, st.acc[tau], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------------------
// Quad-block tile (turbo4 and turbo8 with G <= 4, a ring of at least four slots): the pairing
// above taken to four 16-token blocks, the halves of two consecutive tiles. Column n = G j + h
// (j = 0..3; n >= 4 G repeats column n mod 4 G); lane group gg carries block gg in the query
// operand; MFMA m (0..7) covers dimensions [16 m, 16 m + 16) of all four blocks, so eight MFMAs
// per digit cover 64 tokens, as in the paired layout, while a lane holds 4 scores per 64 tokens.
// PV runs per tile, block j's weights in the k slots of tile j >> 1, half j & 1.
// ---------------------------------------------------------------------------------------
struct QuadLane {
  int jn;      // token block of this lane's column (0..3)
  int hn;      // query head of this lane's column
  int ne;      // the lane's effective column, G jn + hn
};

__device__ __forceinline__ QuadLane quad_lane(int lane, int G) {
  const int n = lane & 15;
  const int ne = n < 4 * G ? n : n % (4 * G);
  return QuadLane{ne / G, ne % G, ne};
}

template <int DT> struct QuadK;
template <> struct QuadK<4> { v4i k[4]; };   // the lane's token row: 16 B per 32 dims
template <> struct QuadK<8> { v4i k[8]; };   // 16 B per 16 dims
template <> struct QuadK<3> { v4i k[1]; };   // never used: turbo3 and turbo2 have no quad layout
template <> struct QuadK<2> { v4i k[1]; };   // (kQuadOk)

template <int DT>
__device__ __forceinline__ void read_quad_k(QuadK<DT>& t, const uint8_t* slot0, const uint8_t* slot1, int lane) {
  using S = Stage<DT>;
  const int gg = lane >> 4, tk = lane & 15;
  const uint8_t* kh = ((gg >> 1) ? slot1 : slot0) + (gg & 1) * S::kHalf;   // block gg, token tk
  if constexpr (DT == 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) t.k[c] = *reinterpret_cast<const v4i*>(kh + 16 * (tk + 16 * c));
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) t.k[m] = *reinterpret_cast<const v4i*>(kh + 1024 * (m & 1) + 16 * (tk + 16 * (m >> 1)));
  }
}

template <int DT>
__device__ __forceinline__ void quad_qk(const QuadK<DT>& t, const v4i (&qq)[8][kDigits], v4i (&s)[kDigits]) {
#pragma unroll
  for (int k = 0; k < kDigits; ++k) s[k] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    v4i a;
    if constexpr (DT == 4) {
      const uint32_t x0 = (uint32_t)t.k[m >> 1][2 * (m & 1)], x1 = (uint32_t)t.k[m >> 1][2 * (m & 1) + 1];
      a = v4i{(int)((x0 << 4) & 0xf0f0f0f0u), (int)(x0 & 0xf0f0f0f0u), (int)((x1 << 4) & 0xf0f0f0f0u),
              (int)(x1 & 0xf0f0f0f0u)};
    } else {
      a = t.k[m];
    }
#pragma unroll
    for (int k = 0; k < kDigits; ++k) s[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qq[m][k], s[k], 0, 0, 0);
  }
}

// The lane's V words of one tile (as laid out in the slot: transposed, dimension-major).
template <int DT> using QuadV = std::conditional_t<DT == 4, int, v2i>[8];

template <int DT>
__device__ __forceinline__ void read_tile_v(QuadV<DT>& v, const uint8_t* slot, int lane) {
  using S = Stage<DT>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (DT == 4)
        v[4 * h + r] = *reinterpret_cast<const int*>(slot + (2 + h) * S::kHalf + 256 * r + 4 * lane);
      else
        v[4 * h + r] = *reinterpret_cast<const v2i*>(slot + (2 + h) * S::kHalf + 512 * r + 8 * lane);
    }
  }
}

// V operand of one tile as fp16 subnormals and the PV MFMAs of that tile against A = (Ahi, Alo).
template <int DT>
__device__ __forceinline__ void tile_pv(const QuadV<DT>& tv, v8h Ahi, v8h Alo, WaveState& st) {
  struct {
    std::conditional_t<DT == 4, int, v2i> v[8];
  } t;
#pragma unroll
  for (int j = 0; j < 8; ++j) t.v[j] = tv[j];
  const v8h Bb = __builtin_bit_cast(v8h, make_uint4(0x00800080u, 0x00800080u, 0x00800080u, 0x00800080u));
  st.accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bb, st.accb, 0, 0, 0);
  st.accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bb, st.accb, 0, 0, 0);
  uint32_t e[8], o[8];
  if constexpr (DT == 4) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t x = (uint32_t)t.v[j];
      e[j] = ((x << 4) & 0xf0f0f0f0u) ^ 0x80808080u;   // even dims, (c + 8) << 4
      o[j] = (x & 0xf0f0f0f0u) ^ 0x80808080u;          // odd dims
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e[j] = (uint32_t)t.v[j][0] ^ 0x80808080u;     // c + 128
      o[j] = (uint32_t)t.v[j][1] ^ 0x80808080u;
    }
  }
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) {
    const uint32_t* src;
    int i;
    if constexpr (DT == 8) {
      src = tau < 4 ? e : o;
      i = tau & 3;
    } else {
      src = (tau & 1) ? o : e;
      i = tau >> 1;
    }
    const uint32_t sel = (uint32_t)i | (0x0cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0cu << 24);
    const v8h B = __builtin_bit_cast(v8h, make_uint4(perm(src[1], src[0], sel), perm(src[3], src[2], sel),
                                                     perm(src[5], src[4], sel), perm(src[7], src[6], sel)));
    st.acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, B, st.acc[tau], 0, 0, 0);
    st.acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, B, st.acc[tau], 0, 0, 0);
  }
}

// Everything a lane reads from the two slots of a 64-token group, so that the slots can be
// refilled before the group is processed.
template <int DT> struct QuadData {
  QuadK<DT> k;
  QuadV<DT> v[2];   // per tile
  v2i ksw, vsw;     // K and V scales of tokens 4 gg + r of block jn
};

// Tiles in slot0 (tokens 0..31) and slot1 (32..63; all masked when absent).
template <int DT>
__device__ __forceinline__ void read_quad(QuadData<DT>& d, const uint8_t* slot0, const uint8_t* slot1,
                                          const QuadLane& ql, int lane) {
  using S = Stage<DT>;
  read_quad_k<DT>(d.k, slot0, slot1, lane);
  const uint8_t* ss = ((ql.jn >> 1) ? slot1 : slot0) + 4 * S::kHalf + 32 * (ql.jn & 1) + 8 * (lane >> 4);
  d.ksw = *reinterpret_cast<const v2i*>(ss);
  d.vsw = *reinterpret_cast<const v2i*>(ss + 64);
  read_tile_v<DT>(d.v[0], slot0, lane);
  read_tile_v<DT>(d.v[1], slot1, lane);
}

// One 64-token group, from registers.
template <int DT, typename Refill>
__device__ __forceinline__ void process_quad(const QuadData<DT>& d, WaveState& st, const v4i (&qq)[8][kDigits],
                                             float qs, int lim, bool full, const QuadLane& ql, int G,
                                             int lane, Refill&& refill) {
  const int gg = lane >> 4;
  v4i s[kDigits];
  quad_qk<DT>(d.k, qq, s);
  refill();   // as for a pair tile
  const v2i ksw = d.ksw, vsw = d.vsw;
  const uint32_t ks[4] = {(uint32_t)ksw[0], (uint32_t)ksw[0] >> 16, (uint32_t)ksw[1], (uint32_t)ksw[1] >> 16};
  uint32_t sv[4] = {(uint32_t)vsw[0] & 0xffffu, (uint32_t)vsw[0] >> 16, (uint32_t)vsw[1] & 0xffffu,
                    (uint32_t)vsw[1] >> 16};
  float y[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    y[r] = __builtin_fmaf(half_lo(ks[r]), digit_sum(s[0][r], s[1][r], s[2][r]), 0.f);
  }
  if (!full) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = 16 * ql.jn + r < lim;
      y[r] = ok ? y[r] : -INFINITY;
      sv[r] = ok ? sv[r] : 0u;    // unwritten or absent slots may hold anything
    }
  }
  const uint32_t smax = max(max(sv[0], sv[1]), max(sv[2], sv[3]));
  const float ymax = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
  float mx = __builtin_fmaf(ymax, qs, (float)(smax >> 10));
  if (__builtin_expect(__any(mx > st.m + kLazy), 0)) {
    // head maximum over the lanes of head hn: columns hn + G j (j = 0..3), all lane groups
    // The source lanes are recomputed here from an opaque copy of the lane id: hoisted out of the
    // tile loop, their divisions by G would hold registers the loop lacks (and be spilled, their
    // reloads draining the ring's loads).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int base = ln & 48, J4 = 4 * G, n = ln & 15;
    const int ne = n < J4 ? n : n % J4;
    mx = fmaxf(mx, __shfl(mx, base | ((ne + G) % J4)));
    mx = fmaxf(mx, __shfl(mx, base | ((ne + 2 * G) % J4)));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool up = mx > st.m + kLazy;
    const float f = up ? __builtin_amdgcn_exp2f(st.m - mx) : 1.f;
    st.m = up ? mx : st.m;
    st.l *= f;
    const int g4 = (ln >> 4) * 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nr = g4 + r;
      const int ner = nr < J4 ? nr : nr % J4;
      const float fr = __shfl(f, ner % G);
#pragma unroll
      for (int tau = 0; tau < 8; ++tau) st.acc[tau][r] *= fr;
      st.accb[r] *= fr;
    }
  }
  const float nref = kWeightExp - st.m;
  float pw[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(y[r], qs, nref));
    st.l += pr;
    pw[r] = __builtin_fmaf(half_lo(sv[r]), pr, 0.f);
  }
  const auto h01 = __builtin_amdgcn_cvt_pkrtz(pw[0], pw[1]);
  const auto h23 = __builtin_amdgcn_cvt_pkrtz(pw[2], pw[3]);
  const auto l01 = __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf((float)h01[0], -1.f, pw[0]),
                                              __builtin_fmaf((float)h01[1], -1.f, pw[1]));
  const auto l23 = __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf((float)h23[0], -1.f, pw[2]),
                                              __builtin_fmaf((float)h23[1], -1.f, pw[3]));
  const uint32_t hi01 = __builtin_bit_cast(uint32_t, h01), hi23 = __builtin_bit_cast(uint32_t, h23);
  const uint32_t lo01 = __builtin_bit_cast(uint32_t, l01), lo23 = __builtin_bit_cast(uint32_t, l23);
#pragma unroll
  for (int tl = 0; tl < 2; ++tl) {
    const bool a = ql.jn == 2 * tl, c = ql.jn == 2 * tl + 1;
    const v8h Ahi = __builtin_bit_cast(v8h, make_uint4(a ? hi01 : 0u, a ? hi23 : 0u, c ? hi01 : 0u, c ? hi23 : 0u));
    const v8h Alo = __builtin_bit_cast(v8h, make_uint4(a ? lo01 : 0u, a ? lo23 : 0u, c ? lo01 : 0u, c ? lo23 : 0u));
    tile_pv<DT>(d.v[tl], Ahi, Alo, st);
  }
}

// Tokens row b attends to: its context length (decode), or start + b + 1 for query b of a
// prefill chunk (causal; every row reads the chunk's sequence's block-table row).
__device__ __forceinline__ int row_context(const DecodeParams& p, int b) {
  return p.ctx_base > 0 ? min(p.ctx_base + b, p.max_context_len) : min(p.context_lens[b], p.max_context_len);
}

// In-place unnormalized FWHT of `rows` rows of 128 floats in LDS, by one wave.
__device__ __forceinline__ void fwht_wave(float (*x)[D + 4], int rows, int lane) {
  for (int h = 1; h < D; h <<= 1) {
    __syncthreads();   // one wave per workgroup: orders the LDS stages
    for (int k = lane; k < rows * 64; k += 64) {
      const int j = k >> 6, r = k & 63;
      const int i = ((r / h) * 2 * h) + (r % h);
      const float a = x[j][i], b = x[j][i + h];
      x[j][i] = a + b;
      x[j][i + h] = a - b;
    }
  }
  __syncthreads();
}

// One wave per work unit (split, kv head, sequence): the wave walks the unit's 32-token tiles
// in order, keeping kDepth of them in flight, and finishes the unit alone (no cross-wave merge,
// no barrier in the loop).
// Waves per SIMD the register budget is sized for: deep rings (4+ slots) are only picked when
// at most two waves share a SIMD; turbo8's 8 KB slots keep even its two-slot rings at about two
// waves per SIMD through the LDS, so it takes the two-wave budget at every depth.
template <int DT, int DEPTH>
constexpr int kWavesPerEu = DT == 0 ? 1 : (DT == kFp8 || DT == 8 ? 2 : (DEPTH >= 4 ? 2 : 3));

// DEPTH: tiles in flight per wave on the staged path (LDS slots); chosen at launch from how
// many waves share a compute unit, so that the LDS of the resident waves holds as many tiles
// in flight as it can.
template <int DT, int DEPTH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEu<DT, DEPTH>)))
void decode_split_kernel(DecodeParams p) {
  // Workgroups after the units append the rows of other sequences (xa): the hardware dispatches
  // them last, so they run as the units finish, on SIMDs the units' tail leaves idle.
  if (p.x_groups > 0) {
    const uint32_t nunits = (uint32_t)p.nsplits * (uint32_t)p.hkv * (((uint32_t)p.batch + p.qt - 1u) / p.qt);
    if (blockIdx.x >= nunits) {
      codec::append_passes<DT>(p.xa, blockIdx.x - nunits, (uint32_t)p.x_groups, threadIdx.x);
      return;
    }
  }
  // Work unit of this wave. Workgroups go to the eight XCDs round-robin by id (XCD = id mod 8).
  // The kv heads of one (split, sequence) share an XCD, whose L2 then fetches each line of a
  // page once for all of them (a page's kv-head blocks are adjacent but not line aligned).
  // With a batch that is a multiple of 8, split s of sequence b goes to XCD (b + s) mod 8, and
  // within an XCD first splits come first: every sequence is spread over all XCDs, every XCD
  // gets the same number of (long) first splits, and those start first. Otherwise (the
  // leftover ids too) units map in (sequence, split) order.
  // A unit's rows: row block b (p.qt consecutive rows: sequences of a decode, where qt = 1, or
  // queries of a prefill chunk).
  int split, kvh, b;
  int unit_tps = p.tokens_per_split;   // tokens per partition of this unit's sequence
  const uint32_t nblocks = ((uint32_t)p.batch + (uint32_t)p.qt - 1u) / (uint32_t)p.qt;
  {
    const uint32_t id = blockIdx.x, hkv = (uint32_t)p.hkv;
    const uint32_t units = (uint32_t)p.nsplits * hkv * nblocks;
    const uint32_t full = units / (8u * hkv) * (8u * hkv);
    if ((nblocks & 7u) == 0) {
      const uint32_t xcd = id & 7u, slot = id >> 3;
      kvh = (int)(slot % hkv);
      const uint32_t r = slot / hkv, per = nblocks >> 3;
      split = (int)(r / per);
      b = (int)(8u * (r % per) + ((xcd - (uint32_t)split) & 7u));
    } else {
      uint32_t group;
      if (id < full) {
        const uint32_t slot = id >> 3;
        kvh = (int)(slot % hkv);
        group = slot / hkv * 8u + (id & 7u);
      } else {
        kvh = (int)(id % hkv);
        group = id / hkv;
      }
      split = (int)(group % (uint32_t)p.nsplits);
      b = (int)(group / (uint32_t)p.nsplits);
    }
    if (p.seq_tps) {
      // a length-aware plan: this slot runs the unit of its pair, or nothing
      const int2 e = reinterpret_cast<const int2*>(p.seq_order)[id];
      if (e.x < 0 || (uint32_t)e.x >= units) return;
      kvh = (int)((uint32_t)e.x % hkv);
      const uint32_t r = (uint32_t)e.x / hkv;
      split = (int)(r % (uint32_t)p.nsplits);
      b = (int)(r / (uint32_t)p.nsplits);
      unit_tps = e.y;
    } else if (p.seq_order) {
      if (p.nsplits > 1) {
        // a unit plan (xq_decode_plan with several partitions): this slot runs unit
        // (b nsplits + split) hkv + kvh, or nothing (-1, or an entry outside the units)
        const int u = p.seq_order[id];
        if (u < 0 || (uint32_t)u >= units) return;
        kvh = (int)((uint32_t)u % hkv);
        const uint32_t r = (uint32_t)u / hkv;
        split = (int)(r % (uint32_t)p.nsplits);
        b = (int)(r / (uint32_t)p.nsplits);
      } else {
        // a host plan may hand this slot another sequence (long and short ones sharing a SIMD)
        // (clamped: an entry outside the batch, outside the contract, still indexes the batch's
        // arrays)
        b = min(max(p.seq_order[b], 0), p.batch - 1);
      }
    }
  }
  const int lane = threadIdx.x;
  // Columns of the unit's MFMA tiles: c = t Gq + h is head h (of the kv head's Gq) of row
  // b0 + t. A decode has one row (G = Gq); a prefill packs 16 / Gq query tokens of the chunk.
  const int Gq = p.group;
  const int qh0 = kvh * Gq;
  const int b0 = b * p.qt;
  if (b0 >= p.batch) return;   // (the grid has no such unit)
  const int nrow = min(p.qt, p.batch - b0);
  const int G = nrow * Gq;
  auto qrow = [&](int c) -> int64_t {   // row of column c in q, out and the partials
    return (int64_t)(b0 + c / Gq) * p.hq + qh0 + c % Gq;
  };
  // The split's block-table window (at most kMaxSplitPages entries from its first page, within
  // the row's max_pages) is loaded before the context length is known, so the two loads overlap;
  // entries past the context are loaded but never used.
  static_assert(kMaxSplitPages <= 128, "two registers of block-table entries");
  int btw0 = 0, btw1 = 0;
  {
    const int lpw = (split * unit_tps) >> p.page_shift;
    const int32_t* row = p.block_tables + (int64_t)b0 * p.bt_stride + lpw;
    const int nwin = min(kMaxSplitPages, p.maxp - lpw);
    if (lane < nwin) btw0 = row[lane];
    if (lane + 64 < nwin) btw1 = row[lane + 64];
  }
  const int L = row_context(p, b0 + nrow - 1);   // the unit's longest row (its last)
  if (L <= 0) {
    if (split == 0)
      for (int i = lane; i < G * D; i += kThreads) p.out[qrow(i >> 7) * D + (i & 127)] = 0.f;
    return;
  }
  const int tps = unit_tps;
  const int tok_begin = split * tps;
  if (tok_begin >= L) return;
  const int tok_end = min(L, tok_begin + tps);
  const int nsplit_b = (L + tps - 1) / tps;
  // causal limits of a prefill: this lane's column attends to tok_end_c tokens of the split; every
  // column of a tile ending by tok_end_min is full
  const int col0 = threadIdx.x & 15;
  const int tok_end_c = min(tok_end, row_context(p, b0 + min(col0, G - 1) / Gq));
  const int tok_end_min = min(tok_end, row_context(p, b0));

  // Fused append (decode rows only): the wave of the sequence's last split encodes the step's new
  // K and V rows of its kv head into slot L - 1 (lanes 0..15 the K row, 16..31 the V row, as the
  // append kernel would) and waits until the stores are done before it loads the tile holding
  // that slot. On the staged path with more tiles than the first DEPTH - 1 staged ones, this runs
  // after those are issued (their loads and the new rows' overlap); otherwise first of all.
  const bool fuse = p.k_new != nullptr && split == nsplit_b - 1;
  uint4 new_raw = make_uint4(0u, 0u, 0u, 0u);   // this lane's 8 elements of the new K (or V) row
  int new_page = 0;
  auto load_new_row = [&]() __attribute__((always_inline)) {
    new_page = p.block_tables[(int64_t)b0 * p.bt_stride + ((L - 1) >> p.page_shift)];
    if (lane < 32)
      new_raw = *reinterpret_cast<const uint4*>((lane >= 16 ? p.v_new : p.k_new) +
                                                ((int64_t)b0 * p.hkv + kvh) * D + (lane & 15) * 8);
  };
  auto store_new_row = [&]() __attribute__((always_inline)) {
    if (lane < 32) {
      uint8_t* block = const_cast<uint8_t*>(lane >= 16 ? p.v_pool : p.k_pool) + (int64_t)new_page * p.page_stride +
                       (int64_t)kvh * p.block_bytes;
      codec::encode_row<DT>(new_raw, lane & 15, block, (L - 1) & (p.page_size - 1), p.page_size);
    }
  };
  const int ntiles = (tok_end - tok_begin + 31) >> 5;
  const bool by_left = p.nsplits > 1;   // issue priority from the tiles left
  const bool fuse_late = fuse && Stage<DT>::kOn && ntiles > DEPTH - 1;
  if (fuse) load_new_row();   // ahead of every cache load, so that waiting for it waits for nothing else
  if (fuse && !fuse_late) {
    store_new_row();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // the staging ring and the epilogue's output rows (plus 64 per-lane sums) share one LDS buffer
  constexpr int kOutBytes = kMaxGroup * (D + 4) * 4 + kThreads * 4;
  constexpr int kRingBytes = DEPTH * Stage<DT>::kSlot;
  constexpr int kSmemBytes = kOutBytes > kRingBytes ? kOutBytes : kRingBytes;
  static_assert(kOutBytes >= kQueryLds, "query rows fit the output rows' LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  auto ob = reinterpret_cast<float (*)[D + 4]>(smem);

  const int col = lane & 15, g = lane >> 4;

  // ---- query operands ---------------------------------------------------------------------
  // turbo types: the wave rotates and quantizes its G query rows itself (rotate_query_lane); the
  // rows arrive by LDS DMA ahead of the first tiles, so the work overlaps their latency
  // (paired and quad layouts: decode only, all columns sharing one row)
  const bool pair = kPairOk<DT> && G <= kPairMaxGroup && p.qt == 1;
  const bool quad = kQuadOk<DT> && pair && DEPTH >= 4 && G <= 4;   // the quad-block layout (pair too)
  const PairLane pl = pair_lane(lane, G);
  const QuadLane ql = quad_lane(lane, G);
  v4i qi[2][kDigits] = {};
  v4i qj[4][kDigits] = {};
  v4i qq[8][kDigits] = {};
  v8bf qb[4] = {};
  float qs = 0.f;
  auto issue_query = [&](uint8_t* qa) __attribute__((always_inline)) {   // G rows of 256 B to qa
    // row t of the unit: Gq rows of 256 B, contiguous in q, to qa + t Gq 256 (1 KB an instruction)
    for (int t = 0; t < nrow; ++t) {
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(p.q + qrow(t * Gq) * D), (short)0, Gq * 256, kBufferConfig);
      for (int i = 0; i < (Gq + 3) >> 2; ++i)
        if (16 * lane + 1024 * i < Gq * 256)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(qa + t * Gq * 256 + 1024 * i), 16, 16 * lane,
                                                   1024 * i, 0, 0);
    }
  };
  auto load_query = [&](uint8_t* qa) __attribute__((always_inline)) {    // after the rows have landed in qa
    float* qsc = reinterpret_cast<float*>(qa + kQueryScaleOff);
    if (G <= 4) {
      QueryLane<8> qr;
      if (lane < 16 * G) {
        rotate_query_lane<DT, 8>(qa, lane >> 4, lane & 15, p.softmax_scale, qr);
        if (pair) write_query_digits<DT, true, 8>(qr, qa, qsc, lane >> 4, lane >> 4, lane & 15);
        else write_query_digits<DT, false, 8>(qr, qa, qsc, lane >> 4, lane >> 4, lane & 15);
      }
    } else if (G <= 8) {
      QueryLane<16> qr;
      if (lane < 8 * G) {
        rotate_query_lane<DT, 16>(qa, lane >> 3, lane & 7, p.softmax_scale, qr);
        if (pair) write_query_digits<DT, true, 16>(qr, qa, qsc, lane >> 3, lane >> 3, lane & 7);
        else write_query_digits<DT, false, 16>(qr, qa, qsc, lane >> 3, lane >> 3, lane & 7);
      }
    } else {
      // more than kQPhaseRows columns (one-block layout): every lane rotates its rows first; the
      // digits of heads 0..7 are written, read as operands by their columns, then overwritten by
      // those of heads 8 and up
      QueryLane<32> qr;
      const int h = lane >> 2;
      if (lane < 4 * G) rotate_query_lane<DT, 32>(qa, h, lane & 3, p.softmax_scale, qr);
      for (int ph = 0; ph * kQPhaseRows < G; ++ph) {
        if (lane < 4 * G && h / kQPhaseRows == ph)
          write_query_digits<DT, false, 32>(qr, qa, qsc, h, h - ph * kQPhaseRows, lane & 3);
        __syncthreads();
        if (col < G && col / kQPhaseRows == ph) {
          const v4i* s = reinterpret_cast<const v4i*>(qa + (col - ph * kQPhaseRows) * kQRowBytes + 32 * kDigits * g);
#pragma unroll
          for (int k = 0; k < kDigits; ++k) {
            qi[0][k] = s[k];
            qi[1][k] = s[kDigits + k];
          }
          qs = qsc[col];
        }
        // the operand reads complete before the next phase overwrites the digits, or a later DMA
        // refills this LDS
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
      }
      return;
    }
    __syncthreads();
    if (quad) {
      // block-diagonal query operand: lane group g carries token block g
      if (ql.jn == g) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const v4i* s = reinterpret_cast<const v4i*>(qa + ql.hn * kQRowBytes + (m >> 1) * 32 * kDigits +
                                                      16 * kDigits * (m & 1));
#pragma unroll
          for (int k = 0; k < kDigits; ++k) qq[m][k] = s[k];
        }
      }
      qs = qsc[ql.hn];
    } else if (pair) {
      // block-diagonal query operand: lane group g carries token block g >> 1
      if (pl.jn == pl.kb) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const v4i* s = reinterpret_cast<const v4i*>(qa + pl.hn * kQRowBytes + m * 32 * kDigits + 16 * kDigits * pl.kp);
#pragma unroll
          for (int k = 0; k < kDigits; ++k) qj[m][k] = s[k];
        }
      }
      qs = qsc[pl.hn];
    } else if (col < G) {
      const v4i* s = reinterpret_cast<const v4i*>(qa + col * kQRowBytes + 32 * kDigits * g);
#pragma unroll
      for (int k = 0; k < kDigits; ++k) {
        qi[0][k] = s[k];
        qi[1][k] = s[kDigits + k];
      }
      qs = qsc[col];
    }
    // the operand reads complete before a later DMA may refill this LDS
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  if constexpr (kBf16Mma<DT>) {
    if (col < G) {
      const int64_t row = qrow(col);
      const v8bf* s = reinterpret_cast<const v8bf*>(p.q + row * D + 32 * g);
      qb[0] = s[0]; qb[1] = s[1]; qb[2] = s[2]; qb[3] = s[3];
      qs = p.softmax_scale * kLog2e;
    }
  } else if constexpr (!Stage<DT>::kOn) {
    issue_query(smem);
    wait_vm<0>();
    load_query(smem);
  }

  WaveState st;
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) st.acc[tau] = v4f{0.f, 0.f, 0.f, 0.f};
  st.accb = v4f{0.f, 0.f, 0.f, 0.f};
  st.m = kNoRef;
  st.l = 0.f;

  // ---- main loop: tiles 0 .. ntiles-1 of the unit, kDepth in flight --------------------------
  constexpr int R = Codec<DT>::kRow;
  const int ps = p.page_size;
  const int last_page = (L - 1) >> p.page_shift;
  const int64_t head_off = (int64_t)kvh * p.block_bytes;
  const LaneOffsets lo = lane_offsets<DT>(col, g);
  const int lp0 = tok_begin >> p.page_shift;     // tok_begin is page aligned

  // Page lookup and descriptors. The unit's block-table entries (a split spans at most
  // kMaxSplitPages = 128 pages) sit in two VGPRs, entry lp0 + i in lane i % 64 of register
  // i / 64, and come back with readlane: a page costs no memory round trip. Pools below 4 GiB
  // (fast form): one descriptor per pool, based at this kv head's block of page 0, serves the
  // whole unit and the page's byte offset rides in the instructions' offsets. Larger pools: a
  // descriptor per page block (reads past the block return zero).
  const bool fast = p.pool_bytes <= (int64_t)0xFFFFFFFF;
  const uint32_t pool_rec = (uint32_t)(p.pool_bytes - head_off);
  const __amdgpu_buffer_rsrc_t k_pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.k_pool + head_off), (short)0, (int)pool_rec, kBufferConfig);
  const __amdgpu_buffer_rsrc_t v_pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.v_pool + head_off), (short)0, (int)pool_rec, kBufferConfig);
  const int nrec = (int)p.block_bytes;
  auto addr = [&](auto kFast, int t0, HalfAddr (&a)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int th = t0 + 16 * h;
      const int lp = min(th >> p.page_shift, last_page);   // never read a table entry past the context
      const int slot = th & (ps - 1);
      const int i = lp - lp0;
      // both registers read, one kept: no branch
      const int p0 = __builtin_amdgcn_readlane(btw0, i & 63), p1 = __builtin_amdgcn_readlane(btw1, i & 63);
      const int phys = i < 64 ? p0 : p1;
      if constexpr (decltype(kFast)::value) {
        const uint32_t base = (uint32_t)phys * (uint32_t)p.page_stride;
        a[h].k = k_pool_rsrc;
        a[h].v = v_pool_rsrc;
        a[h].row = (int)(base + (uint32_t)(slot * R));
        a[h].scale = (int)(base + (uint32_t)(ps * R + 2 * slot));
      } else {
        const int64_t off = (int64_t)phys * p.page_stride + head_off;
        a[h].k = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.k_pool + off), (short)0, nrec, kBufferConfig);
        a[h].v = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.v_pool + off), (short)0, nrec, kBufferConfig);
        a[h].row = slot * R;
        a[h].scale = ps * R + 2 * slot;
      }
    }
  };
  auto run = [&](const Tile<DT>& t, int i) __attribute__((always_inline)) {
    const int t0 = tok_begin + 32 * i;
    process_tile<DT>(t, st, qi, qb, qs, tok_end_c - t0 - 4 * g, tok_end - t0 - 4 * g, t0 + 32 <= tok_end_min, col, g);
  };
  auto main_loop = [&](auto kFast, auto kPair) __attribute__((always_inline)) {
    if constexpr (Stage<DT>::kOn) {
      // slot i % DEPTH holds tile i
      using S = Stage<DT>;
      static_assert((DEPTH - 1) * S::kOps <= kMaxVmcnt, "vmcnt field is 6 bits");
      const DmaOffsets dof = dma_offsets<DT>(lane);
      auto stage = [&](int i, int slot) __attribute__((always_inline)) {   // slot = i % DEPTH
        HalfAddr a[2];
        addr(kFast, tok_begin + 32 * i, a);
        stage_tile<DT, decltype(kFast)::value>(smem + slot * S::kSlot, a, dof, lane);
      };
      auto next_slot = [](int slot) { return slot + 1 == DEPTH ? 0 : slot + 1; };
      std::conditional_t<decltype(kPair)::value, PairTile<DT>, Tile<DT>> tile;
      // the query rows go to the last ring slot, which the loop first fills with tile DEPTH - 1
      uint8_t* qa = smem + (DEPTH - 1) * S::kSlot;
      issue_query(qa);
      // Tiles 0 .. DEPTH - 2 go to their slots beside the query rows (last slot); loads complete
      // in issue order, so the rows are in once at most the staged tiles' loads are pending.
      // After the query is prepared its slot takes tile DEPTH - 1. A step reads its tiles from
      // LDS into registers, issues their QK products, then waits for the reads and refills the
      // freed slots (the paired and quad layouts; the one-block layout refills before its math),
      // so DEPTH tiles are in flight while it computes.
      for (int i = 0; i < DEPTH - 1 && i < ntiles; ++i) stage(i, i);
      // the new rows' stores go out behind the first tiles (the extra operations only make the
      // count-based waits below stricter); they are complete before any later tile is staged
      if (fuse_late) store_new_row();
      wait_tiles<S::kOps, 0, DEPTH - 1>(min(DEPTH - 1, ntiles));
      load_query(qa);   // ends with its LDS reads complete
      if (fuse_late) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (DEPTH - 1 < ntiles) stage(DEPTH - 1, DEPTH - 1);
      // While tiles it .. it + DEPTH - 1 all exist, the number of tiles staged after the ones a
      // step reads is fixed and the wait takes a constant; only the last steps count down.
      if constexpr (kQuadOk<DT> && decltype(kPair)::value && DEPTH >= 4) {
        if (quad) {
          // two tiles per step, in slots cur and next_slot(cur)
          int cur = 0;
          for (int it = 0; it < ntiles; it += 2) {
            if (by_left) issue_priority(ntiles - it);
            // tiles it, it + 1 are in once at most the tiles staged after them (it + 2 ..
            // it + DEPTH - 1) are outstanding
            if (it + DEPTH - 1 < ntiles) wait_vm<(DEPTH - 2) * S::kOps>();
            else wait_tiles<S::kOps, 0, DEPTH - 1>(max(0, ntiles - 2 - it));
            const int nxt = next_slot(cur);
            QuadData<DT> qd;
            read_quad<DT>(qd, smem + cur * S::kSlot, smem + nxt * S::kSlot, ql, lane);
            // the freed slots are refilled once the reads are complete, after the step's QK
            // products are issued
            auto refill = [&]() __attribute__((always_inline)) {
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
              if (it + DEPTH < ntiles) stage(it + DEPTH, cur);
              if (it + DEPTH + 1 < ntiles) stage(it + DEPTH + 1, nxt);
            };
            const int t0 = tok_begin + 32 * it;
            process_quad<DT>(qd, st, qq, qs, tok_end - t0 - 4 * g, t0 + 64 <= tok_end, ql, G, lane, refill);
            cur = next_slot(nxt);
          }
          return;
        }
      }
      int cur = 0;   // slot of tile it
      for (int it = 0; it < ntiles; ++it) {
        if (by_left) issue_priority(ntiles - it);
        // this tile is in once at most the tiles staged after it (it + 1 .. it + DEPTH - 1) are
        // outstanding
        if (it + DEPTH - 1 < ntiles) wait_vm<(DEPTH - 1) * S::kOps>();
        else wait_tiles<S::kOps, 0, DEPTH - 1>(ntiles - 1 - it);
        const int rs = cur;   // the slot read
        auto refill = [&]() __attribute__((always_inline)) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          if (it + DEPTH < ntiles) stage(it + DEPTH, rs);
        };
        cur = next_slot(cur);
        if constexpr (decltype(kPair)::value) {
          read_slot_pair<DT>(tile, smem + rs * S::kSlot, lane, pl);
          // the freed slot is refilled once the reads are complete, after the QK products are
          // issued
          const int t0 = tok_begin + 32 * it;
          process_pair_tile<DT>(tile, st, qj, qs, tok_end - t0 - 4 * g, t0 + 32 <= tok_end, pl, G, lane, refill);
        } else {
          read_slot<DT>(tile, smem + rs * S::kSlot, lane);
          refill();
          run(tile, it);
        }
      }
    } else {
      constexpr int kDepth = kDepthOf<DT>;
      auto fetch = [&](Tile<DT>& t, int i) __attribute__((always_inline)) {
        HalfAddr a[2];
        addr(kFast, tok_begin + 32 * i, a);
        load_tile<DT>(t, a, lo);
      };
      // buffer i % kDepth holds tile i
      Tile<DT> tb[kDepth];
#pragma unroll
      for (int d = 0; d < kDepth - 1; ++d)
        if (d < ntiles) fetch(tb[d], d);
      for (int it = 0; it < ntiles;) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
          if (by_left) issue_priority(ntiles - it);
          const int ahead = it + kDepth - 1;
          if (ahead < ntiles) fetch(tb[(d + kDepth - 1) % kDepth], ahead);
          run(tb[d], it);
          if (++it >= ntiles) break;
        }
      }
    }
  };
  if constexpr (kPairOk<DT>) {
    if (pair) {
      if (fast) main_loop(std::true_type{}, std::true_type{});
      else main_loop(std::false_type{}, std::true_type{});
    } else {
      if (fast) main_loop(std::true_type{}, std::false_type{});
      else main_loop(std::false_type{}, std::false_type{});
    }
  } else {
    if (fast) main_loop(std::true_type{}, std::false_type{});
    else main_loop(std::false_type{}, std::false_type{});
  }

  const float unit = (float)(1 << Codec<DT>::kVShift);
  if (pair) {
    // ---- finish a paired (J = 2) or quad (J = 4) block unit: rows n + G j of the product are
    // head n's block sums; the normaliser of head n is the sum over the lanes of those columns --
    const int J = quad ? 4 : 2;
    float* lsum = reinterpret_cast<float*>(smem + kMaxGroup * (D + 4) * 4);
    __syncthreads();   // the ring is drained (the last tile waited for everything): reuse it
    lsum[lane] = st.l;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r < J * G) {
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) ob[4 * g + r][8 * col + tau] = (st.acc[tau][r] - st.accb[r]) * unit;
      }
    __syncthreads();
    auto head_l = [&](int h) {
      float l = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        for (int j = 0; j < J; ++j) l += lsum[16 * q + G * j + h];
      return l;
    };
    auto head_acc = [&](int h, int d) {
      float a = 0.f;
      for (int j = 0; j < J; ++j) a += ob[G * j + h][d];
      return a;
    };
    if (nsplit_b == 1) {
      for (int k = lane; k < G * D; k += kThreads) {
        const int h = k >> 7, d = k & 127;
        ob[h][d] = head_acc(h, d) / head_l(h);
      }
      fwht_wave(ob, G, lane);
      for (int k = lane; k < G * D; k += kThreads) p.out[qrow(k >> 7) * D + (k & 127)] = ob[k >> 7][k & 127] * kRotC;
    } else {
      for (int k = lane; k < G * D; k += kThreads) {
        const int h = k >> 7, d = k & 127;
        float* part = p.partials + (qrow(h) * p.nsplits + split) * kPartialStride;
        part[4 + d] = head_acc(h, d);
      }
      if (lane < G) {   // lane n < G: column n is head n, block 0
        float* part = p.partials + (qrow(lane) * p.nsplits + split) * kPartialStride;
        part[0] = st.m;
        part[1] = head_l(lane);
      }
    }
    return;
  }

  // ---- finish the unit: combine the four lanes of each head ------------------------------
  st.l += __shfl_xor(st.l, 16);
  st.l += __shfl_xor(st.l, 32);
  if (nsplit_b == 1) {
    // out = H (acc / l); lane (g, c) holds heads 4g + r, dimensions 8c + tau
    float lh[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lh[r] = __shfl(st.l, 4 * g + r);
    __syncthreads();   // the ring is drained (the last tile waited for everything): reuse it
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r < G) {
        const float inv = 1.f / lh[r];
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) ob[4 * g + r][8 * col + tau] = (st.acc[tau][r] - st.accb[r]) * unit * inv;
      }
    if constexpr (kRotated<DT>) {
      fwht_wave(ob, G, lane);
      for (int k = lane; k < G * D; k += kThreads) p.out[qrow(k >> 7) * D + (k & 127)] = ob[k >> 7][k & 127] * kRotC;
    } else {
      __syncthreads();
      for (int k = lane; k < G * D; k += kThreads) p.out[qrow(k >> 7) * D + (k & 127)] = ob[k >> 7][k & 127];
    }
  } else {
    // partials (m, l, acc) of this split, in the rotated space
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r < G) {
        float* part = p.partials + (qrow(4 * g + r) * p.nsplits + split) * kPartialStride;
        float v[8];
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) v[tau] = (st.acc[tau][r] - st.accb[r]) * unit;
        reinterpret_cast<float4*>(part + 4 + 8 * col)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(part + 4 + 8 * col)[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    if (g == 0 && col < G) {
      float* part = p.partials + (qrow(col) * p.nsplits + split) * kPartialStride;
      part[0] = st.m;
      part[1] = st.l;
    }
  }
}

// Merge split partials of one (sequence, q head) and rotate back. THREADS = 32 * groups:
// thread (s0 = t / 32, d4 = t % 32) sums dimensions 4 d4 .. 4 d4 + 3 over splits s0,
// s0 + groups, ..., eight splits per step with their loads issued together (128 threads for a
// few splits, 512 for many; 1024 threads measured slower on 256 splits).
template <int DT, int kCombThreads>
__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(DecodeParams p) {
  constexpr int kCombGroups = kCombThreads / 32;
  const int qh = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x;
  // the split count of b's unit (its last row's), which the split kernel used for every row
  const int L = row_context(p, min(p.batch - 1, (b / p.qt) * p.qt + p.qt - 1));
  const int tps = p.seq_tps ? p.seq_tps[b] : p.tokens_per_split;
  const int ns = (L + tps - 1) / tps;
  if (ns <= 1) return;  // written by the split kernel
  const float* part = p.partials + ((int64_t)b * p.hq + qh) * p.nsplits * kPartialStride;
  __shared__ float4 accs[kCombGroups][32];
  __shared__ float lsum[kCombGroups];
  __shared__ float msum[kCombGroups];
  __shared__ __attribute__((aligned(16))) float o[D];

  // One pass: each group of 32 threads merges its splits into a running (m, l, acc) by
  // log-sum-exp, kU splits' partials loaded together (every load of a step in flight at once: the
  // merge is a chain of dependent rounds of loads); the groups are merged at the end.
  constexpr int kU = 8;
  const int s0 = t >> 5, d4 = t & 31;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float l = 0.f, mt = -INFINITY;
  for (int sb = s0; sb < ns; sb += kU * kCombGroups) {
    float ms[kU], ls[kU];
    float4 a[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = sb + u * kCombGroups;
      const float* ps = part + (int64_t)(s < ns ? s : sb) * kPartialStride;
      ms[u] = s < ns ? ps[0] : -INFINITY;
      ls[u] = ps[1];
      a[u] = reinterpret_cast<const float4*>(ps + 4)[d4];
    }
    // split sb < ns is real, so mn is finite; the first step scales the empty state by 0
    float mn = mt;
#pragma unroll
    for (int u = 0; u < kU; ++u) mn = fmaxf(mn, ms[u]);
    const float fo = __builtin_amdgcn_exp2f(mt - mn);
    acc.x *= fo; acc.y *= fo; acc.z *= fo; acc.w *= fo;
    l *= fo;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float f = (ms[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[u] - mn);
      acc.x += a[u].x * f; acc.y += a[u].y * f; acc.z += a[u].z * f; acc.w += a[u].w * f;
      l += ls[u] * f;   // the same for all 32 lanes of the group
    }
    mt = mn;
  }
  accs[s0][d4] = acc;
  if (d4 == 0) {
    lsum[s0] = l;
    msum[s0] = mt;
  }
  __syncthreads();
  if (t < D) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kCombGroups; ++k) M = fmaxf(M, msum[k]);   // group 0 holds split 0
    float a = 0.f, lt = 0.f;
#pragma unroll
    for (int k = 0; k < kCombGroups; ++k) {
      const float f = msum[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(msum[k] - M);
      const float4 v = accs[k][t >> 2];
      a += ((t & 3) == 0 ? v.x : (t & 3) == 1 ? v.y : (t & 3) == 2 ? v.z : v.w) * f;
      lt += lsum[k] * f;
    }
    o[t] = a / lt;
  }
  float* outp = p.out + ((int64_t)b * p.hq + qh) * D;
  __syncthreads();
  if constexpr (kRotated<DT>) {
    // the inverse rotation on 16 lanes, eight elements each (the transform's stage order)
    if (t < 16) {
      float r[1][8];
      const float4 x0 = reinterpret_cast<const float4*>(o)[2 * t], x1 = reinterpret_cast<const float4*>(o)[2 * t + 1];
      r[0][0] = x0.x; r[0][1] = x0.y; r[0][2] = x0.z; r[0][3] = x0.w;
      r[0][4] = x1.x; r[0][5] = x1.y; r[0][6] = x1.z; r[0][7] = x1.w;
      codec::fwht_row<16>(r, t);
      float4* d4 = reinterpret_cast<float4*>(outp + 8 * t);
      d4[0] = make_float4(r[0][0] * kRotC, r[0][1] * kRotC, r[0][2] * kRotC, r[0][3] * kRotC);
      d4[1] = make_float4(r[0][4] * kRotC, r[0][5] * kRotC, r[0][6] * kRotC, r[0][7] * kRotC);
    }
  } else {
    if (t < D) outp[t] = o[t];
  }
}

// Work units of a call: (split, kv head, block of qt rows).
inline int64_t unit_count(const DecodeParams& p) {
  return (int64_t)p.nsplits * p.hkv * (((int64_t)p.batch + p.qt - 1) / p.qt);
}

// Ring depth for the staged path: the units are spread over 256 compute units; with w of them
// resident per CU (at most 12: three waves per SIMD), the LDS holds 160 KB / (w * slot) slots.
template <int DT>
int pick_depth(const DecodeParams& p) {
  if constexpr (!Stage<DT>::kOn) {
    return 3;
  } else {
    const int64_t units = unit_count(p);
    const int64_t per_cu = std::min<int64_t>(12, std::max<int64_t>(1, (units + 255) / 256));
    const int64_t slots = kLdsPerCu / (per_cu * Stage<DT>::kSlot);
    const int64_t cap = kMaxVmcnt / Stage<DT>::kOps + 1;
    const int64_t d = std::min<int64_t>(slots, cap);
    // Deep rings cost occupancy (two waves per SIMD at most) and pay only for a single wave per
    // SIMD, or for turbo8's quad layout at up to two. Measured on MI355X with two or three waves
    // per SIMD, the loads in flight are not what limits a unit: two slots run as fast as three or
    // four (turbo4, 256 sequences of up to 1,024 tokens: 40.7 us with two slots, 41.4 with three,
    // 42.7 with four in the quad layout; turbo3, one 262,144-token sequence in 256 partitions:
    // 80.0, 81.0, 81.2), six run far slower (57 and 116 us), and turbo8 gains from its quad
    // layout (32 sequences of 8,192 tokens: 109 us with four slots, 116 with two or three).
    if (per_cu <= 4 && d >= 4) return d >= 8 ? 8 : d >= 6 ? 6 : 4;
    if (DT == 8 && per_cu <= 8 && d >= 4) return 4;
    return 2;
  }
}

// Waves per SIMD the launch runs at once when all its workgroups are resident: the register
// budget's target, or fewer where the LDS of one compute unit holds fewer rings.
template <int DT>
int waves_per_simd(const DecodeParams& p) {
  const int depth = Stage<DT>::kOn ? (p.fixed_splits ? 3 : pick_depth<DT>(p)) : 3;
  const int regs = depth >= 4 ? kWavesPerEu<DT, 4> : kWavesPerEu<DT, 3>;
  constexpr int kOut = kMaxGroup * (D + 4) * 4 + kThreads * 4;
  const int ring = depth * Stage<DT>::kSlot;
  const int by_lds = (kLdsPerCu / std::max(kOut, ring)) / 4;
  return std::max(1, std::min(regs, by_lds));
}

template <int DT, int DEPTH>
void launch_split(const DecodeParams& p, hipStream_t stream) {
  const int64_t grid = unit_count(p) + p.x_groups;
  hipLaunchKernelGGL((decode_split_kernel<DT, DEPTH>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
}

template <int DT>
void combine_dt(const DecodeParams& p, hipStream_t stream) {
  if (p.nsplits > 32 && !p.fixed_splits)
    hipLaunchKernelGGL((decode_combine_kernel<DT, 512>), dim3(p.hq, p.batch), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_combine_kernel<DT, 128>), dim3(p.hq, p.batch), dim3(128), 0, stream, p);
}

// With fixed partitions (batch-invariant mode) the kernel variants do not depend on the batch:
// a three-slot ring (the paired/one-block layouts, never the quad one, whose blocking of the
// softmax differs) and the 128-thread combine, so a sequence's output depends only on its own
// inputs and the partition size.
template <int DT>
hipError_t launch_dt(const DecodeParams& p, hipStream_t stream) {
  if constexpr (Stage<DT>::kOn) {
    switch (p.fixed_splits ? 3 : pick_depth<DT>(p)) {
      case 8: launch_split<DT, (Stage<DT>::kOps * 7 <= kMaxVmcnt ? 8 : 6)>(p, stream); break;
      case 6: launch_split<DT, 6>(p, stream); break;
      case 4: launch_split<DT, 4>(p, stream); break;
      case 3: launch_split<DT, 3>(p, stream); break;
      default: launch_split<DT, 2>(p, stream); break;
    }
  } else {
    launch_split<DT, 3>(p, stream);
  }
  if (p.nsplits > 1) combine_dt<DT>(p, stream);
  return hipGetLastError();
}

}  // namespace

int decode_waves_per_simd(int dtype, const DecodeParams& p) {
  switch (dtype) {
    case 0: return waves_per_simd<0>(p);
    case 8: return waves_per_simd<8>(p);
    case 4: return waves_per_simd<4>(p);
    case 3: return waves_per_simd<3>(p);
    case 2: return waves_per_simd<2>(p);
    case kFp8: return waves_per_simd<kFp8>(p);
    default: return 1;
  }
}

hipError_t launch_combine(int dtype, const DecodeParams& p, hipStream_t stream) {
  switch (dtype) {
    case 0: combine_dt<0>(p, stream); break;
    case 8: combine_dt<8>(p, stream); break;
    case 4: combine_dt<4>(p, stream); break;
    case 3: combine_dt<3>(p, stream); break;
    case 2: combine_dt<2>(p, stream); break;
    case kFp8: combine_dt<kFp8>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, const DecodeParams& p, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_dt<0>(p, stream);
    case 8: return launch_dt<8>(p, stream);
    case 4: return launch_dt<4>(p, stream);
    case 3: return launch_dt<3>(p, stream);
    case 2: return launch_dt<2>(p, stream);
    case kFp8: return launch_dt<kFp8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xq
