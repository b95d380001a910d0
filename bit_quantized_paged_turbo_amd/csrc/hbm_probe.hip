// Streaming-read reference for the decode's roofline (a measurement aid, not part of the
// attention method): how fast this GPU's HBM delivers bytes when nothing but reading happens,
// both as one sequential stream and as 1 KiB blocks gathered through a page table, the access
// pattern of the decode (a turbo4 page block of 16 rows holds 1 KiB of codes).
//
// One 64-lane wave reads one 1 KiB chunk per instruction (16 B a lane, non-temporal, like the
// decode's cache reads); waves walk the blocks in a grid stride, four chunks in flight per lane.
// Every lane XORs what it reads and stores the result only if it equals a value the host picks,
// so the loads cannot be dropped and (in practice) nothing is written.
#include "xq_internal.h"

#include <algorithm>

namespace xq {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kChunk = 1024;   // bytes one wave reads per instruction

__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const uint8_t* buf, uint32_t total, int chunk_shift,
                                                                 int64_t stride, const int32_t* order, uint32_t* sink,
                                                                 uint32_t flag) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
  const uint32_t nwaves = (gridDim.x * kProbeThreads) >> 6;
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  v4u acc = {0u, 0u, 0u, 0u};
  // chunk c of the call is chunk c & (2^chunk_shift - 1) of block c >> chunk_shift
  for (uint32_t c0 = wave * 4; c0 < total; c0 += nwaves * 4) {
    v4u r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t c = min(c0 + u, total - 1);
      const uint32_t blk = c >> chunk_shift;
      const int64_t page = order ? (int64_t)order[blk] : (int64_t)blk;
      const uint8_t* src = buf + page * stride + (int64_t)(c & ((1u << chunk_shift) - 1)) * kChunk + 16 * lane;
      r[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= r[u];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == flag) sink[0] = x;
}

}  // namespace

hipError_t launch_hbm_probe(const uint8_t* buf, int64_t n_blocks, int32_t block_bytes, int64_t stride,
                            const int32_t* order, uint32_t* sink, hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  int shift = 0;
  while ((kChunk << shift) < block_bytes) ++shift;   // block_bytes = 1 KiB x 2^shift
  const int64_t total = n_blocks << shift;           // < 2^31 (checked by the caller)
  // enough waves to fill every SIMD several times over (256 CUs, 4 SIMDs each)
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(256 * 16, (total + 15) / 16));
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream, buf, (uint32_t)total,
                     shift, stride, order, sink, 0x9e3779b9u);
  return hipGetLastError();
}

}  // namespace xq
