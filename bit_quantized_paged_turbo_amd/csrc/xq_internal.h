// Internal interface between the C ABI (xq_abi.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xq {

constexpr int kHeadDim = 128;
constexpr int kMaxGroup = 16;         // query heads per kv head: the 16 columns of one MFMA tile
constexpr int kPartialStride = 132;   // floats per (seq, q head, split) partial: m, l, pad, acc[128]
constexpr int kMaxSplitPages = 128;   // pages per split: the block-table window of a decode wave

constexpr int kFp8 = 16;              // cache-type value of the E4M3 cache (not a code width)

// Bytes of one stored code row for a dtype (bf16: 256, fp8: 128).
inline constexpr int row_code_bytes(int dtype) { return dtype == 0 ? 256 : dtype == kFp8 ? 128 : 16 * dtype; }
// Whether rows carry an fp16 scale after the page's code rows (the turbo types).
inline constexpr bool has_scales(int dtype) { return dtype != 0 && dtype != kFp8; }

inline constexpr int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Workspace of one decode call: the split partials (only with more than one split).
struct WorkspaceLayout {
  int64_t part_off, part_bytes;      // float [batch][hq][nsplits][kPartialStride]  (nsplits > 1)
  int64_t total;
};

inline WorkspaceLayout workspace_layout(int dtype, int64_t batch, int64_t hq, int64_t nsplits) {
  (void)dtype;
  WorkspaceLayout w{};
  w.part_off = 0;
  w.part_bytes = nsplits > 1 ? align256(batch * hq * nsplits * kPartialStride * 4) : 0;
  w.total = w.part_off + w.part_bytes;
  return w;
}

struct AppendParams {
  const uint16_t* k_new;        // bf16 [n_tokens][hkv][128]
  const uint16_t* v_new;
  const int32_t* token_seq;     // [n_tokens]
  const int32_t* token_pos;     // [n_tokens]
  const int32_t* block_tables;  // [num_seqs][maxp]
  uint8_t* k_pool;
  uint8_t* v_pool;
  int64_t page_stride;          // bytes
  int64_t block_bytes;          // bytes
  int32_t n_tokens;
  int32_t hkv;
  int32_t page_size;
  int32_t maxp;
};

struct DecodeParams {
  const uint16_t* q;            // bf16 [batch][hq][128]
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;  // [batch][maxp]
  const int32_t* context_lens;  // [batch]
  float* out;                   // [batch][hq][128]
  float* partials;              // workspace: [batch][hq][nsplits][kPartialStride] (nsplits > 1)
  int64_t page_stride;
  int64_t block_bytes;
  int64_t pool_bytes;           // bytes of each pool (num_pages * page_stride)
  int32_t batch;
  int32_t hq;
  int32_t hkv;
  int32_t group;                // hq / hkv, 1..kMaxGroup
  int32_t page_size;
  int32_t page_shift;           // log2(page_size)
  int32_t maxp;
  int32_t tokens_per_split;     // multiple of page_size and of 32
  int32_t nsplits;              // splits of the longest sequence (grid x)
  int32_t max_context_len;      // context_lens are clamped to this
  float softmax_scale;
  int32_t fixed_splits;         // 1: partitions fixed by the caller; kernel variants chosen
                                // independently of the batch, so results are batch invariant
  int32_t bt_stride;            // block-table entries between rows (maxp; 0: one shared row)
  int32_t ctx_base;             // 0: row b attends to context_lens[b] tokens; > 0: to
                                // ctx_base + b tokens (query b of a prefill chunk)
  int32_t qt;                   // rows per work unit: 1 (decode) or 16 / group (prefill)
  const int32_t* seq_order;     // null, or a plan from xq_decode_plan: with one partition per
                                // sequence a permutation of the batch (the slot of sequence b in
                                // the unit order runs sequence seq_order[b]); with several, one
                                // entry per work slot: the unit (b nsplits + split) hkv + kvh that
                                // workgroup id runs, or -1
  const uint16_t* k_new;        // null, or bf16 [batch][hkv][128]: new rows appended at position
  const uint16_t* v_new;        // context_lens[b] - 1 by the wave of b's last split, first
  // Length-aware partitions (xq_decode_plan_balanced): when set, sequence b is cut into
  // partitions of seq_tps[b] tokens, and seq_order holds one pair {unit, tokens per partition}
  // per work slot (unit = (b nsplits + split) hkv + kvh, or -1 for none); tokens_per_split is
  // unused and nsplits is the partitions' stride (at least every sequence's count).
  const int32_t* seq_tps;
  // Rows of other sequences appended by the same launch (a prefill chunk beside the decodes):
  // x_groups workgroups after the decode's units run xa's append passes; none when 0.
  AppendParams xa;
  int32_t x_groups;
};

hipError_t launch_quantize_append(int dtype, const AppendParams& p, hipStream_t stream);
hipError_t launch_decode(int dtype, const DecodeParams& p, hipStream_t stream);
// Merge of split partials (m, l, acc) into the rotated-back outputs: p.nsplits partitions of
// p.tokens_per_split tokens, the partition count of row b being that of the last row of its
// block of p.qt rows; a block with one partition is skipped (its rows are written by the kernel
// that computed them).
hipError_t launch_combine(int dtype, const DecodeParams& p, hipStream_t stream);
// Chunked prefill on the tile kernel (cache types for which prefill_tiled holds): one workgroup
// per (partition, kv head, block of p.qt = prefill_block_queries(group) queries;
// prefill_workgroups of them), then the combine when p.nsplits > 1.
bool prefill_tiled(int dtype);
int prefill_block_queries(int group);
int64_t prefill_workgroups(int32_t n_query, int32_t group, int32_t hkv, int32_t nsplits);
hipError_t launch_prefill(int dtype, const DecodeParams& p, hipStream_t stream);
// Waves of the decode's split kernel resident on one SIMD for the launch launch_decode would make
// with these parameters (the register budget and the LDS of a compute unit).
int decode_waves_per_simd(int dtype, const DecodeParams& p);
// Streaming-read reference: n_blocks blocks of block_bytes (1 KiB times a power of two), block i at
// order[i] * stride (i * stride when order is null).
hipError_t launch_hbm_probe(const uint8_t* buf, int64_t n_blocks, int32_t block_bytes, int64_t stride,
                            const int32_t* order, uint32_t* sink, hipStream_t stream);

}  // namespace xq
