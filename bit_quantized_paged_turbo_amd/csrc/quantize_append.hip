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
// and one of scales per page. Waves walk their passes (K rows, then V rows) with the next
// pass's rows already loading (the rows are streamed once: the loads are non-temporal).
//
// The fp8 cache type (same page, section "Getting a server up: the commands in the README",
// and its compression table: 2x against BF16) stores each bf16 element as the nearest finite
// OCP FP8 E4M3 value, ties to even, saturating at 448: no rotation, no scale.
#include "row_codec.h"

#pragma clang fp contract(off)

namespace xq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Workgroups per launch at most: about four waves per SIMD, what the registers (about 100 a lane)
// keep resident at once; larger appends loop.
constexpr int kMaxBlocks = 1024;

template <int BITS>
__global__ __launch_bounds__(kThreads) void quantize_append_kernel(AppendParams p) {
  // the wave's first pass is the same for its 64 lanes: taken from lane 0, so the pass loop's
  // index arithmetic runs on the scalar unit
  const uint32_t first = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
  codec::append_passes<BITS>(p, first, gridDim.x * kWaves, threadIdx.x & 63);
}

}  // namespace

hipError_t launch_quantize_append(int dtype, const AppendParams& p, hipStream_t stream) {
  if (p.n_tokens <= 0) return hipSuccess;
  const int64_t passes = 2 * (((int64_t)p.n_tokens + codec::kAppendRows - 1) / codec::kAppendRows * p.hkv);
  const int64_t blocks = std::min<int64_t>((passes + kWaves - 1) / kWaves, kMaxBlocks);
  dim3 grid((unsigned)blocks, 1, 1);
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
