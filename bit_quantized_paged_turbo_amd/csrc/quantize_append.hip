// Fused rotate + quantize + pack + page scatter for new K/V rows (gfx950).
//
// Method: "xInfer: Pure-Rust LLM Inference Without a Python Runtime" (hysenlabs.com),
// section "What actually sits between the request and the tokens": every K/V head vector
// is rotated by a Walsh-Hadamard transform and then quantized with a per-head absmax
// scale. Number format fixed by this library (the pages leave it open): fp32 FWHT stages
// h = 1..64 of (a+b, a-b), one multiply by C = fp32(1/sqrt(128)), s16 = fp16_rne(
// min(absmax/qmax, 65504)), c = clamp(rint_half_even(x/s16), +-qmax), bits-wide two's
// complement fields packed little-endian. Codes and scales must be bit-identical to the
// CPU definition: the row encoder (row_codec.h) runs without FP contraction, and its
// reciprocal shortcut falls back to IEEE division wherever it could differ.
//
// Work layout: one row = one (token, kv head) vector of K or V. Four lanes own a row, 32
// elements each, as four 16-byte pieces: piece k of lane l holds elements 8 (l + 4k) .. + 7,
// so each of the four loads reads 64 contiguous bytes per row. Butterfly stages h = 1, 2, 4
// and 32, 64 run inside a lane, h = 8, 16 across the row's lanes (DPP within a quad). A wave
// encodes 16 rows per pass, one kv head of 16 consecutive tokens: a chunk's consecutive
// positions fill consecutive slots of a page, so the pass writes one contiguous run of codes
// and one of scales per page. Waves walk their passes with the next pass's rows already
// loading (the rows are streamed once: the loads are non-temporal). blockIdx.y = 0 encodes K
// rows, 1 V rows.
//
// The fp8 cache type (same page, section "Getting a server up: the commands in the README",
// and its compression table: 2x against BF16) stores each bf16 element as the nearest finite
// OCP FP8 E4M3 value, ties to even, saturating at 448: no rotation, no scale.
#include "row_codec.h"

#pragma clang fp contract(off)

namespace xq {
namespace {

constexpr int kLanesPerRow = 4;
constexpr int kRowsPerPass = 64 / kLanesPerRow;   // rows a wave encodes at once
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Workgroups per launch at most (per K/V half): the two halves' waves, four per SIMD, are about
// what the registers (about 100 a lane) keep resident at once; larger appends loop.
constexpr int kMaxBlocks = 512;

typedef unsigned v4u __attribute__((ext_vector_type(4)));

struct RowIn {
  uint4 raw[kLanesPerRow];   // this lane's four pieces
  int seq, pos;              // the row's token: its sequence and position
};

template <int BITS>
__global__ __launch_bounds__(kThreads) void quantize_append_kernel(AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int l = lane & (kLanesPerRow - 1);      // lane of the row
  const int rw = lane / kLanesPerRow;           // token of the pass's 16
  const uint32_t ntok = (uint32_t)p.n_tokens;   // n_tokens * hkv < 2^28, checked by the caller
  const uint32_t hkv = (uint32_t)p.hkv;
  // pass = 16-token block * hkv + kv head
  const uint32_t npass = (ntok + kRowsPerPass - 1) / kRowsPerPass * hkv;
  const bool is_v = blockIdx.y != 0;
  const uint16_t* src = is_v ? p.v_new : p.k_new;
  uint8_t* pool = is_v ? p.v_pool : p.k_pool;
  const uint32_t stride = gridDim.x * kWaves;
  const int shift = __builtin_ctz((unsigned)p.page_size);

  auto token_of = [&](uint32_t pass) { return pass / hkv * kRowsPerPass + rw; };
  auto load = [&](uint32_t pass, RowIn& in) __attribute__((always_inline)) {
    const uint32_t tok = token_of(pass);
    if (tok < ntok) {
      const uint32_t row = tok * hkv + pass % hkv;
      const uint16_t* s = src + (int64_t)row * kHeadDim + 8 * l;
#pragma unroll
      for (int k = 0; k < kLanesPerRow; ++k) {
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(s + 8 * kLanesPerRow * k));
        in.raw[k] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      in.seq = p.token_seq[tok];
      in.pos = p.token_pos[tok];
    }
  };

  uint32_t pass = blockIdx.x * kWaves + (threadIdx.x >> 6);
  RowIn cur;
  if (pass < npass) load(pass, cur);
  while (pass < npass) {
    const uint32_t tok = token_of(pass);
    const uint32_t head = pass % hkv;
    int page = 0;
    if (tok < ntok) page = p.block_tables[(int64_t)cur.seq * p.maxp + (cur.pos >> shift)];
    // the next pass's rows load while this one is encoded
    const uint32_t next = pass + stride;
    RowIn nxt;
    if (next < npass) load(next, nxt);
    if (tok < ntok) {
      uint8_t* block = pool + (int64_t)page * p.page_stride + (int64_t)head * p.block_bytes;
      codec::encode_row_lanes<BITS, kLanesPerRow>(cur.raw, l, block, cur.pos & (p.page_size - 1), p.page_size);
    }
    cur = nxt;
    pass = next;
  }
}

}  // namespace

hipError_t launch_quantize_append(int dtype, const AppendParams& p, hipStream_t stream) {
  if (p.n_tokens <= 0) return hipSuccess;
  const int64_t passes = ((int64_t)p.n_tokens + kRowsPerPass - 1) / kRowsPerPass * p.hkv;
  const int64_t blocks = std::min<int64_t>((passes + kWaves - 1) / kWaves, kMaxBlocks);
  dim3 grid((unsigned)blocks, 2, 1);
  switch (dtype) {
    case 0: hipLaunchKernelGGL(quantize_append_kernel<0>, grid, dim3(kThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(quantize_append_kernel<8>, grid, dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(quantize_append_kernel<4>, grid, dim3(kThreads), 0, stream, p); break;
    case 3: hipLaunchKernelGGL(quantize_append_kernel<3>, grid, dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(quantize_append_kernel<2>, grid, dim3(kThreads), 0, stream, p); break;
    case kFp8: hipLaunchKernelGGL(quantize_append_kernel<kFp8>, grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace xq
