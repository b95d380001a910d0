// Chunked prefill attention over the paged TurboQuant cache, gfx950: a tile kernel for the many
// queries of one sequence's chunk.
//
// Method: the decode's quantities ("xInfer: Pure-Rust LLM Inference Without a Python Runtime",
// hysenlabs.com, section "What actually sits between the request and the tokens": cached K/V
// rows are Walsh-Hadamard rotated and absmax-quantized per head) for a chunk of queries that
// attend causally to the sequence's cached rows and to their own (infero landing page, section
// "Beyond plain text decode", item "Continuous batching": prefill fills the rest of a step and
// may be split across steps). As in the decode, q.k = (Hq).(Hk): the queries are rotated once,
// scores are taken against the stored rotated rows and the value sum is rotated back.
//
// The decode reads each cache row once per query row, so there the dequantization work per row
// is spread over one sequence's g query heads. A chunk has many queries per cached row, so this
// kernel dequantizes each 64-token K/V tile once per workgroup into LDS as fp16 and lets four
// waves of 2 x 16 (query, head) columns each run both products on the matrix cores from there:
//
//   QK  v_mfma_f32_16x16x32_f16: rows = 16 tokens, columns = 16 (query, head) pairs of one kv
//       head. A K code c is the exact fp16 integer c. The rotated query, scaled by the softmax
//       scale, log2(e) and one power of two per workgroup (its largest element near 2^14), is
//       split into an fp16 high part and the fp16 remainder; both enter the same fp32
//       accumulator, so each element carries about 22 bits. The K scale of the token (times
//       the inverse power of two) multiplies the sum.
//   PV  v_mfma_f32_16x16x32_f16: rows = the 16 columns, k = 32 tokens, columns = 16 dimensions.
//       The weight P' = p * s_v is split into fp16 high (round toward zero) and remainder parts
//       as in the decode, against V codes as exact fp16 integers (transposed in LDS, so a lane's
//       eight k values are one 16-byte read).
//
// Softmax: the decode's lazily moved log2-domain reference per column, tracking score plus the
// largest fp16 exponent field of the tile's s_v (the decode's per-token bound taken per tile), so
// P' stays within fp16 whatever the scales are; the normaliser sum(p) is fp32. States of one query from several partitions are merged by the decode's
// combine kernel (same partial format), which also rotates back; with one partition the
// workgroup normalises, rotates back and stores itself.
//
// Work split: one workgroup per (partition, kv head, block of 8 * (16 / g) queries). Tiles are
// loaded into registers one tile ahead, converted and written to the other half of a two-tile
// LDS buffer, one barrier per tile; a wave skips the tiles none of its queries reaches.
// Workgroups are issued longest causal block first, with the second half of the grid in the
// reverse order, so that the two workgroups a compute unit holds together carry about the mean
// work. (Pairing each block's first half with the mirrored half from the chunk's end, so that
// every workgroup carries the mean work, measured slower on MI355X: 161 against 133 us for a
// 2,048-query chunk, the groups of a wave then running on different tile ranges.) The cache
// types differ only in the tile conversion (load_raw, k_pair, v_pair).
#include "row_codec.h"
#include "xq_internal.h"

#include <type_traits>

namespace xq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// bf16 and fp8 caches hold plain (unrotated, unscaled) rows: K and V tiles are staged as bf16,
// the bf16 query enters QK exactly in one pass, and the output is not rotated back.
template <int DT> constexpr bool kPlain = DT == 0 || DT == kFp8;

// One 16x16x32 matrix-core product on operands held as four dwords: fp16 for the turbo types,
// bf16 for the plain ones.
template <int DT>
__device__ __forceinline__ v4f mma(uint4 a, uint4 b, v4f c) {
  if constexpr (kPlain<DT>)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                   0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

constexpr int D = kHeadDim;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kNC = 2;                       // 16-column groups per wave
constexpr int kTile = 64;                    // tokens per K/V tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRotC = 0x1.6a09e6p-4f;      // fp32 nearest to 1/sqrt(128)
constexpr float kLazy = 8.0f;                // move the reference only when a score beats it by > 2^8
constexpr float kWeightExp = 21.f;           // p = 2^(y - m + 21): P' = p s_v < 2^15 in fp16
constexpr float kNoRef = -1e30f;             // finite initial reference (a fully masked column gets p = 0)

// LDS of one tile: K rows of fp16 codes in the dimension order of k_pos (row stride padded so
// that 16 lanes reading 16 different rows hit distinct banks), V transposed (one row per
// dimension over the tile's tokens in the order of the PV k slots, padded likewise), per token
// the K scale (times the inverse query power of two) and s_v, and the largest fp16 exponent
// field of the tile's s_v.
constexpr int kKRow = 2 * D + 16;
constexpr int kVRow = 2 * kTile + 16;
constexpr int kVOff = kTile * kKRow;
constexpr int kSOff = kVOff + D * kVRow;
constexpr int kStage = kSOff + 2 * kTile * 4 + 16;
constexpr int kLds = 2 * kStage;
constexpr int kQWave = kNC * 16 * D * 2 * 2;      // per wave: hi and lo fp16 query operands
constexpr int kORow = D + 4;
constexpr int kOWave = kNC * 16 * kORow * 4;      // per wave: normalised output rows (fp32)
static_assert(kWaves * kQWave <= kLds && kWaves * kOWave <= kLds, "query and output areas fit the tile buffer");

// Position of dimension 8 j + e (e < 8) in a K row: 8 j + 2 (e & 3) + (e >> 2). The unpack below
// makes fp16 pairs of the codes (e, e + 4) of each group of eight dimensions, so the row holds
// each group as 0 4 1 5 2 6 3 7; the query operand is laid out the same way.
__device__ __forceinline__ int k_pos(int e) { return 2 * (e & 3) + (e >> 2); }

// Position of tile token t in a V row: the PV k slots 8 g .. 8 g + 7 of MFMA j are tokens
// 32 j + 4 g + r (slots 8 g + r) and 32 j + 16 + 4 g + r (slots 8 g + 4 + r): where the QK
// product leaves lane (g, c)'s scores.
__device__ __forceinline__ int v_pos(int t) {
  return 32 * (t >> 5) + 8 * ((t >> 2) & 3) + 4 * ((t >> 4) & 1) + (t & 3);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// fp16 pair (c0, c1) of two biased codes n = c + 2^(bits - 1) in bits 0..7 and 16..23 of x (its
// other bits zero): 0x6400 | n is the fp16 value 1024 + n, so one packed subtraction gives the
// codes exactly.
template <int DT>
__device__ __forceinline__ uint32_t code_pair(uint32_t x) {
  constexpr _Float16 off = (_Float16)(1024.f + (float)(1 << (DT - 1)));
  const h2 v = __builtin_bit_cast(h2, x | 0x64006400u) - h2{off, off};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t bfe(uint32_t x, int off, int w) { return __builtin_amdgcn_ubfe(x, off, w); }
__device__ __forceinline__ uint32_t align(uint32_t hi, uint32_t lo, int shift) {
  return __builtin_amdgcn_alignbit(hi, lo, shift);
}

// Byte i of lo into bits 0..7 and byte i of hi into bits 16..23, zeros elsewhere.
constexpr uint32_t pair_sel(int i) {
  return (uint32_t)i | (0x0cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0cu << 24);
}

// ---- one tile's raw bytes as one thread loads them ----------------------------------------
// K: thread t holds dimensions 32 (t >> 6) .. + 31 of token t & 63 (4 bits bytes). V: dimensions
// 8 (t >> 4) .. + 7 of tokens 4 (t & 15) .. + 3 (bits bytes each; turbo3's three bytes start at
// any byte, so the two dwords around them are read). Threads t < 64: the fp16 K and V scales of
// token t. Tokens at or past the partition's end read as zero codes and zero scales. The lanes
// of a wave thus write 16 different K rows and, for V, 16 different 8-byte pieces of one
// dimension row, so that the LDS writes meet no bank conflict.
template <int DT> struct Raw {
  static constexpr int kRow = row_code_bytes(DT);                     // code bytes of a row
  static constexpr int kK = kRow / 16;                                // dwords of K per thread
  static constexpr int kV = DT == 0 ? 4 : DT == 8 || DT == kFp8 || DT == 3 ? 2 : 1;
  uint32_t k[kK];      // a quarter row of K
  uint32_t v[4][kV];   // per token: bf16 four dwords, turbo8 and fp8 two, turbo4 one, turbo3 the
                       // dwords around its three bytes, turbo2 one halfword
  uint32_t s;
};

struct Src {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* bt;        // the sequence's block-table row
  int64_t page_stride;
  int64_t head_off;         // kv head * block bytes
  int page_shift, page_mask, scale_off;
};

// Byte offset of token t's page block (of this kv head) in the pools.
__device__ __forceinline__ int64_t block_addr(const Src& s, int t) {
  return (int64_t)s.bt[t >> s.page_shift] * s.page_stride + s.head_off;
}

template <int DT>
__device__ __forceinline__ void load_raw(Raw<DT>& R, const Src& s, int T0, int t_end, int tid) {
  constexpr int kRow = Raw<DT>::kRow;
  const int tk = T0 + (tid & 63);
  const int64_t kb = tk < t_end ? block_addr(s, tk) : 0;
  const int kslot = tk & s.page_mask;
  {
    const uint8_t* src = s.k_pool + kb + kslot * kRow + (kRow / 4) * (tid >> 6);
    if constexpr (Raw<DT>::kK >= 8) {
#pragma unroll
      for (int u = 0; u < Raw<DT>::kK / 4; ++u) {
        const uint4 a = tk < t_end ? reinterpret_cast<const uint4*>(src)[u] : make_uint4(0u, 0u, 0u, 0u);
        R.k[4 * u] = a.x; R.k[4 * u + 1] = a.y; R.k[4 * u + 2] = a.z; R.k[4 * u + 3] = a.w;
      }
    } else if constexpr (DT == 4) {
      const uint4 a = tk < t_end ? *reinterpret_cast<const uint4*>(src) : make_uint4(0u, 0u, 0u, 0u);
      R.k[0] = a.x; R.k[1] = a.y; R.k[2] = a.z; R.k[3] = a.w;
    } else if constexpr (DT == 3) {
      const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
      R.k[0] = tk < t_end ? s32[0] : 0u;
      R.k[1] = tk < t_end ? s32[1] : 0u;
      R.k[2] = tk < t_end ? s32[2] : 0u;
    } else {
      const uint2 a = tk < t_end ? *reinterpret_cast<const uint2*>(src) : make_uint2(0u, 0u);
      R.k[0] = a.x; R.k[1] = a.y;
    }
  }
  {
    const int t0 = T0 + 4 * (tid & 15);
    const int dg = tid >> 4;
    // the four tokens share a page (pages hold at least 16 tokens and t0 is a multiple of 4)
    const int64_t base = t0 < t_end ? block_addr(s, t0) + (t0 & s.page_mask) * kRow : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = t0 + i < t_end;
      const uint8_t* row = s.v_pool + base + kRow * i;
      if constexpr (DT == 0) {
        const uint4 a = ok ? *reinterpret_cast<const uint4*>(row + 16 * dg) : make_uint4(0u, 0u, 0u, 0u);
        R.v[i][0] = a.x; R.v[i][1] = a.y; R.v[i][2] = a.z; R.v[i][3] = a.w;
      } else if constexpr (DT == 8 || DT == kFp8) {
        const uint2 a = ok ? *reinterpret_cast<const uint2*>(row + 8 * dg) : make_uint2(0u, 0u);
        R.v[i][0] = a.x;
        R.v[i][1] = a.y;
      } else if constexpr (DT == 4) {
        R.v[i][0] = ok ? *reinterpret_cast<const uint32_t*>(row + 4 * dg) : 0u;
      } else if constexpr (DT == 3) {
        // bytes 3 dg .. 3 dg + 2 lie in dword (3 dg) / 4 and, from byte 2 of it on, the next one
        // (never past the row's last dword: dg = 15 starts at byte 1 of dword 11)
        const int dw = (3 * dg) >> 2;
        const uint32_t* r32 = reinterpret_cast<const uint32_t*>(row);
        R.v[i][0] = ok ? r32[dw] : 0u;
        R.v[i][1] = ok && ((3 * dg) & 3) >= 2 ? r32[dw + 1] : 0u;
      } else {
        R.v[i][0] = ok ? (uint32_t)*reinterpret_cast<const uint16_t*>(row + 2 * dg) : 0u;
      }
    }
  }
  R.s = 0u;
  if (has_scales(DT) && tid < kTile && tk < t_end) {
    const int64_t off = kb + s.scale_off + 2 * kslot;
    R.s = (uint32_t)*reinterpret_cast<const uint16_t*>(s.k_pool + off) |
          ((uint32_t)*reinterpret_cast<const uint16_t*>(s.v_pool + off) << 16);
  }
}

// K: the biased code pair (dimensions 8 j + i, 8 j + i + 4) of the thread's 32 dimensions, j, i < 4.
template <int DT>
__device__ __forceinline__ uint32_t k_pair(const Raw<DT>& R, int j, int i) {
  if constexpr (DT == 8) {
    return perm(R.k[2 * j + 1], R.k[2 * j], pair_sel(i)) ^ 0x00800080u;
  } else if constexpr (DT == 4) {
    return ((R.k[j] ^ 0x88888888u) >> (4 * i)) & 0x000f000fu;
  } else if constexpr (DT == 3) {
    // group j's 24 bits start at bit 24 j of the 96; the top bit of every 3-bit field flipped
    constexpr uint32_t kFlip[3] = {0x24924924u, 0x49249249u, 0x92492492u};
    const uint32_t k0 = R.k[0] ^ kFlip[0], k1 = R.k[1] ^ kFlip[1], k2 = R.k[2] ^ kFlip[2];
    const uint32_t gj = j == 0 ? k0 : j == 1 ? align(k1, k0, 24) : j == 2 ? align(k2, k1, 16) : k2 >> 8;
    return bfe(gj, 3 * i, 3) | (bfe(gj, 3 * i + 12, 3) << 16);
  } else {
    // bytes (dimensions 0-3, 8-11, 4-7, 12-15 of the dword): group j's pair i at bits 8 (j & 1) + 2 i
    const uint32_t y = perm(R.k[j >> 1], R.k[j >> 1], 0x03010200u) ^ 0xaaaaaaaau;
    return (y >> (8 * (j & 1) + 2 * i)) & 0x00030003u;
  }
}

// V: the biased code pair (token 2 u, token 2 u + 1) of dimension 8 dg + e, u < 2, e < 8.
template <int DT>
__device__ __forceinline__ uint32_t v_pair(const Raw<DT>& R, int u, int e, int dg) {
  const int a = 2 * u, b = 2 * u + 1;
  if constexpr (DT == 8) {
    return perm(R.v[b][e >> 2], R.v[a][e >> 2], pair_sel(e & 3)) ^ 0x00800080u;
  } else if constexpr (DT == 4) {
    const uint32_t p = perm(R.v[b][0], R.v[a][0], pair_sel(e >> 1)) ^ 0x00880088u;
    return (p >> (4 * (e & 1))) & 0x000f000fu;
  } else if constexpr (DT == 3) {
    const int sh = 8 * ((3 * dg) & 3);
    const uint32_t ga = align(R.v[a][1], R.v[a][0], sh) ^ 0x924924u;
    const uint32_t gb = align(R.v[b][1], R.v[b][0], sh) ^ 0x924924u;
    return bfe(ga, 3 * e, 3) | (bfe(gb, 3 * e, 3) << 16);
  } else {
    const uint32_t z = (R.v[a][0] | (R.v[b][0] << 16)) ^ 0xaaaaaaaau;
    return (z >> (2 * e)) & 0x00030003u;
  }
}

template <int DT>
__device__ __forceinline__ void write_stage(uint8_t* st, const Raw<DT>& R, int tid, float inv_s) {
  uint8_t* kdst = st + (tid & 63) * kKRow + 64 * (tid >> 6);
  const int dg = tid >> 4;
  const int p0 = v_pos(4 * (tid & 15));
  if constexpr (kPlain<DT>) {
    // K: the quarter row as bf16, dimensions in order (fp8 widened exactly, two bytes a convert)
    uint32_t kb[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      if constexpr (DT == 0) {
        kb[d] = R.k[d];
      } else {
        kb[d] = __builtin_bit_cast(uint32_t, (d & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(R.k[d >> 1], 1.f, true)
                                                     : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(R.k[d >> 1], 1.f, false));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(kdst + 16 * j) = make_uint4(kb[4 * j], kb[4 * j + 1], kb[4 * j + 2], kb[4 * j + 3]);
    // V: dimension e of tokens (0, 1) and (2, 3) as bf16 pairs
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t pr[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if constexpr (DT == 0) {
          pr[u] = perm(R.v[2 * u + 1][e >> 1], R.v[2 * u][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
        } else {
          const uint32_t b = perm(R.v[2 * u + 1][e >> 2], R.v[2 * u][e >> 2],
                                  (uint32_t)(e & 3) | ((uint32_t)(4 + (e & 3)) << 8) | 0x0c0c0000u);
          pr[u] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.f, false));
        }
      }
      *reinterpret_cast<uint2*>(st + kVOff + (8 * dg + e) * kVRow + 2 * p0) = make_uint2(pr[0], pr[1]);
    }
    (void)inv_s;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(kdst + 16 * j) =
          make_uint4(code_pair<DT>(k_pair<DT>(R, j, 0)), code_pair<DT>(k_pair<DT>(R, j, 1)),
                     code_pair<DT>(k_pair<DT>(R, j, 2)), code_pair<DT>(k_pair<DT>(R, j, 3)));
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint2*>(st + kVOff + (8 * dg + e) * kVRow + 2 * p0) =
          make_uint2(code_pair<DT>(v_pair<DT>(R, 0, e, dg)), code_pair<DT>(v_pair<DT>(R, 1, e, dg)));
    if (tid < kTile) {   // wave 0
      float* sc = reinterpret_cast<float*>(st + kSOff);
      const _Float16 ks = __builtin_bit_cast(_Float16, (uint16_t)(R.s & 0xffffu));
      const _Float16 vs = __builtin_bit_cast(_Float16, (uint16_t)(R.s >> 16));
      sc[tid] = (float)ks * inv_s;
      sc[kTile + tid] = (float)vs;
      // the largest fp16 exponent field of the tile's V scales
      int e = (int)((R.s >> 26) & 31u);
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) e = max(e, __shfl_xor(e, m));
      if (tid == 0) sc[2 * kTile] = (float)e;
    }
  }
}

struct Col {
  int q;       // query index in the chunk
  int head;    // query head
  bool ok;
};

// Workgroup (partition, kv head, block) holds QB = 8 (16 / g) consecutive queries: wave w's
// column c of group n is query blk QB + (2 w + n) (16 / g) + c / g, head kvh g + c % g.
template <int DT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_tile_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float wmax[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int G = p.group, qt = 16 / G, QB = p.qt;
  const int nblk = (p.batch + QB - 1) / QB;

  // ---- unit: the longest causal blocks first; the second half of the grid in reverse order, so
  // that the two workgroups a compute unit holds together carry about the mean work ------------
  const int P = gridDim.x, half = (P + 1) >> 1;
  const int u = (int)blockIdx.x < half ? (int)blockIdx.x : P - 1 - ((int)blockIdx.x - half);
  const int per_blk = p.nsplits * p.hkv;
  const int blk = nblk - 1 - u / per_blk;
  const int split = (u % per_blk) / p.hkv, kvh = u % p.hkv;
  const int q0 = blk * QB;
  const int ctx_max = p.ctx_base + min(q0 + QB, p.batch) - 1;   // the block's longest context
  const int tps = p.tokens_per_split;
  const int t_begin = split * tps;
  if (t_begin >= ctx_max) return;                        // no token of this partition (and no partial read)
  const int t_end = min(t_begin + tps, ctx_max);
  const int ntiles = (t_end - t_begin + kTile - 1) / kTile;

  auto column = [&](int n, int c) {
    Col r;
    const int i = c / G;
    r.q = q0 + (kNC * w + n) * qt + i;
    r.head = kvh * G + c % G;
    r.ok = i < qt && r.q < p.batch;
    return r;
  };

  // ---- queries: rotate (FWHT), scale, one power of two for the workgroup, fp16 hi/lo (plain
  // caches: the bf16 query rows themselves, read straight into the operand layout) ---------------
  uint4 qh[kNC][4], ql[kNC][4];
  float inv_s = 1.f;
  if constexpr (kPlain<DT>) {
#pragma unroll
    for (int n = 0; n < kNC; ++n) {
      const Col col = column(n, c16);
      const uint16_t* src = p.q + ((int64_t)col.q * p.hq + col.head) * D + 8 * g;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        qh[n][m] = col.ok ? *reinterpret_cast<const uint4*>(src + 32 * m) : make_uint4(0u, 0u, 0u, 0u);
        ql[n][m] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  } else {
  float xr[kNC][4][8];
  float am = 0.f;
  {
    const int c = lane >> 2, k4 = lane & 3;
#pragma unroll
    for (int n = 0; n < kNC; ++n) {
      const Col col = column(n, c);
      const uint16_t* src = p.q + ((int64_t)col.q * p.hq + col.head) * D;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint4 v = col.ok ? *reinterpret_cast<const uint4*>(src + 8 * (k4 + 4 * kk)) : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xr[n][kk][2 * e] = __uint_as_float(a[e] << 16);
          xr[n][kk][2 * e + 1] = __uint_as_float(a[e] & 0xffff0000u);
        }
      }
      codec::fwht_row<4>(xr[n], k4);
      const float f = kRotC * p.softmax_scale * kLog2e;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xr[n][kk][e] *= f;
          am = fmaxf(am, fabsf(xr[n][kk][e]));
        }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
  if (lane == 0) wmax[w] = am;
  __syncthreads();
  am = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // S = 2^(14 - ex) with am < 2^ex: the largest scaled element lies in [2^13, 2^14)
  int ex = (int)((__float_as_uint(am) >> 23) & 255u) - 126;
  ex = am > 0.f && ex < 129 ? max(ex, -85) : 14;
  const float S = __uint_as_float((uint32_t)(127 + 14 - ex) << 23);
  inv_s = __uint_as_float((uint32_t)(127 - 14 + ex) << 23);
  {
    uint8_t* qa = smem + w * kQWave;
    const int c = lane >> 2, k4 = lane & 3;
#pragma unroll
    for (int n = 0; n < kNC; ++n) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        v8h hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = xr[n][kk][e] * S;
          const _Float16 h = (_Float16)x;
          hi[k_pos(e)] = h;
          lo[k_pos(e)] = (_Float16)(x - (float)h);
        }
        uint8_t* row = qa + n * (16 * D * 4) + c * (D * 2);
        *reinterpret_cast<v8h*>(row + 16 * (k4 + 4 * kk)) = hi;
        *reinterpret_cast<v8h*>(row + 16 * D * 2 + 16 * (k4 + 4 * kk)) = lo;
      }
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kNC; ++n)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint8_t* row = qa + n * (16 * D * 4) + c16 * (D * 2) + 2 * (32 * m + 8 * g);
        qh[n][m] = *reinterpret_cast<const uint4*>(row);
        ql[n][m] = *reinterpret_cast<const uint4*>(row + 16 * D * 2);
      }
  }
  }

  // causal limits: column c of group n attends to tokens < ctx_base + its query; the wave's
  // smallest limit (below it no token is masked) and largest (from it all are)
  int lim[kNC];
#pragma unroll
  for (int n = 0; n < kNC; ++n) {
    const Col col = column(n, c16);
    lim[n] = col.ok ? min(p.ctx_base + col.q, t_end) : t_end;
  }
  const int wq0 = q0 + kNC * w * qt;
  const int wq1 = min(q0 + (kNC * w + kNC) * qt, p.batch) - 1;
  const int wave_lo = min(t_end, p.ctx_base + wq0);
  const int wave_hi = wq0 < p.batch ? min(t_end, p.ctx_base + wq1) : t_begin;

  const float qsc = p.softmax_scale * kLog2e;   // plain caches: the score scale (log2 domain)
  Src src;
  src.k_pool = p.k_pool;
  src.v_pool = p.v_pool;
  src.bt = p.block_tables;
  src.page_stride = p.page_stride;
  src.head_off = (int64_t)kvh * p.block_bytes;
  src.page_shift = p.page_shift;
  src.page_mask = p.page_size - 1;
  src.scale_off = p.page_size * Raw<DT>::kRow;

  v4f acc[kNC][8];
  float mref[kNC], lsum[kNC];
#pragma unroll
  for (int n = 0; n < kNC; ++n) {
    mref[n] = kNoRef;
    lsum[n] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[n][t] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  Raw<DT> R;
  load_raw<DT>(R, src, t_begin, t_end, tid);
  __syncthreads();                       // the query operands are read: the buffer is free
  write_stage<DT>(smem, R, tid, inv_s);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int T0 = t_begin + it * kTile;
    if (it + 1 < ntiles) load_raw<DT>(R, src, T0 + kTile, t_end, tid);
    const uint8_t* st = smem + (it & 1) * kStage;
    // The tile's products for both groups, with the causal mask applied (compile-time M) or not.
    auto tile = [&](auto m_t) {
      constexpr bool kMask = decltype(m_t)::value;
      // ---- scores ------------------------------------------------------------------------------
      v4f s[kNC][4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint8_t* kr = st + (16 * h + c16) * kKRow + 16 * g;
        uint4 ka[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) ka[m] = *reinterpret_cast<const uint4*>(kr + 64 * m);
#pragma unroll
        for (int n = 0; n < kNC; ++n) {
          v4f a = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            a = mma<DT>(ka[m], qh[n][m], a);
            if constexpr (!kPlain<DT>) a = mma<DT>(ka[m], ql[n][m], a);
          }
          s[n][h] = a;
        }
      }
      // ---- softmax weights, in place of the scores, one group after the other (a group's scores
      // die as its PV operands are made). The reference tracks score + E, E the largest fp16
      // exponent field of the tile's s_v, so P' = p s_v < 2^15 (as per token in the decode); the
      // K and V scales are read from LDS where they are used. Plain caches: the softmax scale in
      // place of the K scale, no V scale (the decode's bf16 path: bf16 weights need no bound) -----
      const float* sc = reinterpret_cast<const float*>(st + kSOff);
      const float evm = kPlain<DT> ? 0.f : sc[2 * kTile];
      uint4 ahi[kNC][2], alo[kNC][2];
#pragma unroll
      for (int n = 0; n < kNC; ++n) {
        float mx = -INFINITY;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const v4f ks = kPlain<DT> ? v4f{qsc, qsc, qsc, qsc} : *reinterpret_cast<const v4f*>(sc + 16 * h + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float y = s[n][h][r] * ks[r];
            if constexpr (kMask) y = T0 + 16 * h + 4 * g + r >= lim[n] ? -INFINITY : y;
            s[n][h][r] = y;
            mx = fmaxf(mx, y);
          }
        }
        mx += evm;
        if (__builtin_expect(__any(mx > mref[n] + kLazy), 0)) {
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const bool up = mx > mref[n] + kLazy;
          const float f = up ? __builtin_amdgcn_exp2f(mref[n] - mx) : 1.f;
          mref[n] = up ? mx : mref[n];
          lsum[n] *= f;
          float fr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) fr[r] = __shfl(f, 4 * g + r);
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[n][t][r] *= fr[r];
        }
        const float mw = kPlain<DT> ? mref[n] : mref[n] - kWeightExp;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const v4f sv = kPlain<DT> ? v4f{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const v4f*>(sc + kTile + 16 * h + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pe = __builtin_amdgcn_exp2f(s[n][h][r] - mw);
            lsum[n] += pe;
            s[n][h][r] = kPlain<DT> ? pe : pe * sv[r];
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const float a = s[n][2 * j + (kk >> 1)][2 * (kk & 1)], b = s[n][2 * j + (kk >> 1)][2 * (kk & 1) + 1];
            if constexpr (kPlain<DT>) {
              // bf16 high parts (truncation) and the bf16 remainders
              const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
              const float ra = a - __uint_as_float(ua & 0xffff0000u), rb = b - __uint_as_float(ub & 0xffff0000u);
              hi[kk] = perm(ub, ua, 0x07060302u);
              lo[kk] = perm(__float_as_uint(rb), __float_as_uint(ra), 0x07060302u);
            } else {
              const auto h2v = __builtin_amdgcn_cvt_pkrtz(a, b);
              const auto l2v = __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf((float)h2v[0], -1.f, a),
                                                          __builtin_fmaf((float)h2v[1], -1.f, b));
              hi[kk] = __builtin_bit_cast(uint32_t, h2v);
              lo[kk] = __builtin_bit_cast(uint32_t, l2v);
            }
          }
          ahi[n][j] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
          alo[n][j] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
      }
      // ---- PV --------------------------------------------------------------------------------
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint4 vb = *reinterpret_cast<const uint4*>(st + kVOff + (16 * t + c16) * kVRow + 64 * j + 16 * g);
#pragma unroll
          for (int n = 0; n < kNC; ++n) {
            acc[n][t] = mma<DT>(ahi[n][j], vb, acc[n][t]);
            acc[n][t] = mma<DT>(alo[n][j], vb, acc[n][t]);
          }
        }
    };
    if (T0 < wave_hi) {                                  // the wave's queries reach the tile
      if (T0 + kTile > wave_lo) tile(std::true_type{});
      else tile(std::false_type{});
    }
    if (it + 1 < ntiles) write_stage<DT>(smem + ((it + 1) & 1) * kStage, R, tid, inv_s);
    __syncthreads();
  }

  // ---- finish: per column, the normaliser is the sum over the column's four lanes. A block
  // whose longest context fits one partition is finished here (the combine skips it); otherwise
  // this partition's (m, l, acc) go to the workspace ------------------------------------------
  float lc[kNC];
#pragma unroll
  for (int n = 0; n < kNC; ++n) {
    lc[n] = lsum[n] + __shfl_xor(lsum[n], 16);
    lc[n] += __shfl_xor(lc[n], 32);
  }
  if (ctx_max <= tps) {
    // out = H (acc / l) / sqrt(128); lane (g, c) holds columns 4 g + r, dimensions 16 t + c
    float* ob = reinterpret_cast<float*>(smem + w * kOWave);
#pragma unroll
    for (int n = 0; n < kNC; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float inv = 1.f / __shfl(lc[n], 4 * g + r);
#pragma unroll
        for (int t = 0; t < 8; ++t) ob[(16 * n + 4 * g + r) * kORow + 16 * t + c16] = acc[n][t][r] * inv;
      }
    __syncthreads();
    const int c = lane >> 2, k4 = lane & 3;
#pragma unroll
    for (int n = 0; n < kNC; ++n) {
      const Col col = column(n, c);
      float x[4][8];
      const float* row = ob + (16 * n + c) * kORow;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float4 a = *reinterpret_cast<const float4*>(row + 8 * (k4 + 4 * kk));
        const float4 b = *reinterpret_cast<const float4*>(row + 8 * (k4 + 4 * kk) + 4);
        x[kk][0] = a.x; x[kk][1] = a.y; x[kk][2] = a.z; x[kk][3] = a.w;
        x[kk][4] = b.x; x[kk][5] = b.y; x[kk][6] = b.z; x[kk][7] = b.w;
      }
      if constexpr (!kPlain<DT>) codec::fwht_row<4>(x, k4);
      constexpr float rc = kPlain<DT> ? 1.f : kRotC;
      if (col.ok) {
        float* dst = p.out + ((int64_t)col.q * p.hq + col.head) * D;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          float4* d4 = reinterpret_cast<float4*>(dst + 8 * (k4 + 4 * kk));
          d4[0] = make_float4(x[kk][0] * rc, x[kk][1] * rc, x[kk][2] * rc, x[kk][3] * rc);
          d4[1] = make_float4(x[kk][4] * rc, x[kk][5] * rc, x[kk][6] * rc, x[kk][7] * rc);
        }
      }
    }
  } else {
    // partials (m, l, acc) of this partition, in the rotated space, for the combine kernel
#pragma unroll
    for (int n = 0; n < kNC; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const Col col = column(n, 4 * g + r);
        if (col.ok) {
          float* part = p.partials + (((int64_t)col.q * p.hq + col.head) * p.nsplits + split) * kPartialStride;
#pragma unroll
          for (int t = 0; t < 8; ++t) part[4 + 16 * t + c16] = acc[n][t][r];
        }
      }
      const Col col = column(n, c16);
      if (g == 0 && col.ok) {
        float* part = p.partials + (((int64_t)col.q * p.hq + col.head) * p.nsplits + split) * kPartialStride;
        part[0] = mref[n];
        part[1] = lc[n];
      }
    }
  }
}

}  // namespace

bool prefill_tiled(int dtype) {
  return dtype == 8 || dtype == 4 || dtype == 3 || dtype == 2 || dtype == 0 || dtype == kFp8;
}

int prefill_block_queries(int group) { return kWaves * kNC * (16 / group); }

int64_t prefill_workgroups(int32_t n_query, int32_t group, int32_t hkv, int32_t nsplits) {
  const int64_t qb = prefill_block_queries(group);
  return (n_query + qb - 1) / qb * hkv * nsplits;
}

hipError_t launch_prefill(int dtype, const DecodeParams& p, hipStream_t stream) {
  const int64_t grid = prefill_workgroups(p.batch, p.group, p.hkv, p.nsplits);
  switch (dtype) {
    case 8:
      hipLaunchKernelGGL((prefill_tile_kernel<8>), dim3((unsigned)grid), dim3(kThreads), kLds, stream, p);
      break;
    case 4:
      hipLaunchKernelGGL((prefill_tile_kernel<4>), dim3((unsigned)grid), dim3(kThreads), kLds, stream, p);
      break;
    case 3:
      hipLaunchKernelGGL((prefill_tile_kernel<3>), dim3((unsigned)grid), dim3(kThreads), kLds, stream, p);
      break;
    case 2:
      hipLaunchKernelGGL((prefill_tile_kernel<2>), dim3((unsigned)grid), dim3(kThreads), kLds, stream, p);
      break;
    case 0:
      hipLaunchKernelGGL((prefill_tile_kernel<0>), dim3((unsigned)grid), dim3(kThreads), kLds, stream, p);
      break;
    case kFp8:
      hipLaunchKernelGGL((prefill_tile_kernel<kFp8>), dim3((unsigned)grid), dim3(kThreads), kLds, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (p.nsplits > 1) return launch_combine(dtype, p, stream);
  return hipGetLastError();
}

}  // namespace xq
