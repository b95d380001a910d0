// Fused rotate + quantize + pack + page scatter for new K/V rows (gfx950).
//
// Method: "xInfer: Pure-Rust LLM Inference Without a Python Runtime" (hysenlabs.com),
// section "What actually sits between the request and the tokens": every K/V head vector
// is rotated by a Walsh-Hadamard transform and then quantized with a per-head absmax
// scale. Number format fixed by this library (the pages leave it open): fp32 FWHT stages
// h = 1..64 of (a+b, a-b), one multiply by C = fp32(1/sqrt(128)), s16 = fp16_rne(
// min(absmax/qmax, 65504)), c = clamp(rint_half_even(x/s16), +-qmax), bits-wide two's
// complement fields packed little-endian. Codes and scales must be bit-identical to the
// CPU definition: the row encoder (row_codec.h) runs without FP contraction and keeps IEEE
// division.
//
// Work layout: one row = one (token, kv head) vector of K or V. Sixteen lanes own a row,
// eight consecutive elements each (one 16-byte load of bf16). Butterfly stages h = 1, 2, 4
// run inside a lane, h = 8..64 across lanes (partner lane = lane ^ h/8). A 256-thread
// workgroup handles 16 rows of K (blockIdx.y = 0) or V (blockIdx.y = 1); a row's 16 lanes
// store its code bytes as one contiguous 16*bits-byte segment of the page block.
//
// The fp8 cache type (same page, section "Getting a server up: the commands in the README",
// and its compression table: 2x against BF16) stores each bf16 element as the nearest finite
// OCP FP8 E4M3 value, ties to even, saturating at 448: no rotation, no scale.
#include "row_codec.h"

#pragma clang fp contract(off)

namespace xq {
namespace {

constexpr int kRowsPerBlock = 16;
constexpr int kThreads = 256;

template <int BITS>
__global__ __launch_bounds__(kThreads) void quantize_append_kernel(AppendParams p) {
  const int lane16 = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);  // (token, head)
  const int64_t nrows = (int64_t)p.n_tokens * p.hkv;
  if (row >= nrows) return;  // uniform within the 16-lane group
  const bool is_v = blockIdx.y != 0;
  const int tok = (int)(row / p.hkv);
  const int head = (int)(row - (int64_t)tok * p.hkv);

  // the row's load does not depend on the page lookup: issue it first so the two overlap
  const uint16_t* src = (is_v ? p.v_new : p.k_new) + row * kHeadDim + lane16 * 8;
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u rv = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src));
  const uint4 raw = make_uint4(rv[0], rv[1], rv[2], rv[3]);
  const int seq = p.token_seq[tok];
  const int pos = p.token_pos[tok];
  const int page = p.block_tables[(int64_t)seq * p.maxp + pos / p.page_size];
  const int slot = pos % p.page_size;
  uint8_t* block = (is_v ? p.v_pool : p.k_pool) + (int64_t)page * p.page_stride +
                   (int64_t)head * p.block_bytes;

  codec::encode_row<BITS>(raw, lane16, block, slot, p.page_size);
}

}  // namespace

hipError_t launch_quantize_append(int dtype, const AppendParams& p, hipStream_t stream) {
  if (p.n_tokens <= 0) return hipSuccess;
  const int64_t rows = (int64_t)p.n_tokens * p.hkv;
  dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock), 2, 1);
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
