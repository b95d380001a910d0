// C ABI of the TurboQuant paged KV cache: argument validation, split planning and launch.
// Declarations and the full contract are in include/xq.h.
#include "../../include/xq.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <unordered_set>
#include <algorithm>
#include <mutex>
#include <vector>

#include "xq_internal.h"

namespace {

thread_local std::string g_last_error;

xq_status fail(xq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool is_dtype(int32_t d) {
  return d == XQ_KV_BF16 || d == XQ_KV_TURBO8 || d == XQ_KV_TURBO4 || d == XQ_KV_TURBO3 || d == XQ_KV_TURBO2 ||
         d == XQ_KV_FP8;
}
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

xq_status check_layout(const xq_cache_layout* L) {
  if (!L) return fail(XQ_EINVAL, "layout is NULL");
  if (!is_dtype(L->kv_dtype)) return fail(XQ_EINVAL, "kv_dtype %d is not one of 0 (bf16), 8, 4, 3, 2, 16 (fp8)", L->kv_dtype);
  if (L->head_dim != 128) return fail(XQ_EUNSUPPORTED, "head_dim %d: only 128 is supported", L->head_dim);
  if (L->num_kv_heads < 1) return fail(XQ_EINVAL, "num_kv_heads %d < 1", L->num_kv_heads);
  if (!pow2(L->page_size) || L->page_size < 16 || L->page_size > 256)
    return fail(XQ_EINVAL, "page_size %d is not a power of two in [16, 256]", L->page_size);
  if (L->num_pages < 1) return fail(XQ_EINVAL, "num_pages %lld < 1", (long long)L->num_pages);
  return XQ_OK;
}

// ---- XQ_DEBUG: checks of device-array contents -------------------------------------------
// On when the environment variable XQ_DEBUG is set to anything but "" or "0" (read at every
// call). The arrays are copied to host memory on the caller's stream, which the call then
// waits for; a violation of the contract returns XQ_EINVAL and launches nothing.
bool debug_on() {
  const char* e = std::getenv("XQ_DEBUG");
  return e && *e && std::strcmp(e, "0") != 0;
}

xq_status fetch(std::vector<int32_t>& h, const int32_t* d, int64_t n, hipStream_t s) {
  h.resize((size_t)n);
  hipError_t e = hipMemcpyAsync(h.data(), d, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(XQ_EHIP, "XQ_DEBUG copy of a device array: %s", hipGetErrorString(e));
  return XQ_OK;
}

// decode: 0 <= context_lens[b] <= max_context_len, and the block-table entries of the pages
// holding positions below context_lens[b] are page ids in [0, num_pages)
xq_status debug_check_decode(const xq_cache_layout* L, int32_t batch, const int32_t* block_tables,
                             int32_t maxp, const int32_t* context_lens, int32_t max_ctx, hipStream_t s) {
  std::vector<int32_t> cl, bt;
  if (xq_status st = fetch(cl, context_lens, batch, s)) return st;
  if (xq_status st = fetch(bt, block_tables, (int64_t)batch * maxp, s)) return st;
  for (int32_t b = 0; b < batch; ++b) {
    if (cl[b] < 0 || cl[b] > max_ctx)
      return fail(XQ_EINVAL, "XQ_DEBUG: context_lens[%d] = %d is outside [0, max_context_len = %d]", b, cl[b],
                  max_ctx);
    const int32_t pages = (cl[b] + L->page_size - 1) / L->page_size;
    for (int32_t i = 0; i < pages; ++i) {
      const int32_t pg = bt[(size_t)b * maxp + i];
      if (pg < 0 || pg >= L->num_pages)
        return fail(XQ_EINVAL, "XQ_DEBUG: block_tables[%d][%d] = %d is not a page id below num_pages = %lld", b,
                    i, pg, (long long)L->num_pages);
    }
  }
  return XQ_OK;
}

// planned decode: seq_order is a permutation of 0 .. batch - 1.
xq_status debug_check_order(int32_t batch, const int32_t* seq_order, hipStream_t s) {
  std::vector<int32_t> o;
  if (xq_status st = fetch(o, seq_order, batch, s)) return st;
  std::vector<char> seen((size_t)batch, 0);
  for (int32_t i = 0; i < batch; ++i) {
    if (o[i] < 0 || o[i] >= batch || seen[(size_t)o[i]])
      return fail(XQ_EINVAL, "XQ_DEBUG: seq_order[%d] = %d: not a permutation of the batch", i, o[i]);
    seen[(size_t)o[i]] = 1;
  }
  return XQ_OK;
}

// planned decode with several partitions: every entry is -1 or a unit index below `units`, no unit
// appears twice, and every unit with tokens (split < ceil(context_lens[b] / tps)) appears, and
// partition 0 of every sequence (which writes an empty sequence's zero output).
xq_status debug_check_unit_plan(int32_t batch, int32_t hkv, int32_t nsplits, int32_t tps, int32_t max_ctx,
                                const int32_t* context_lens, const int32_t* plan, hipStream_t s) {
  const int64_t units = (int64_t)nsplits * hkv * batch;
  std::vector<int32_t> o, cl;
  if (xq_status st = fetch(o, plan, units, s)) return st;
  if (xq_status st = fetch(cl, context_lens, batch, s)) return st;
  std::vector<char> seen((size_t)units, 0);
  for (int64_t i = 0; i < units; ++i) {
    if (o[i] < -1 || o[i] >= units || (o[i] >= 0 && seen[(size_t)o[i]]))
      return fail(XQ_EINVAL, "XQ_DEBUG: plan[%lld] = %d: not -1 or a unit that appears once", (long long)i, o[i]);
    if (o[i] >= 0) seen[(size_t)o[i]] = 1;
  }
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t L = std::min(std::max(cl[b], 0), max_ctx);
    const int32_t n = std::max(1, (L + tps - 1) / tps);   // partition 0 of an empty sequence writes zeros
    for (int32_t sp = 0; sp < n; ++sp)
      for (int32_t k = 0; k < hkv; ++k)
        if (!seen[((size_t)b * nsplits + sp) * hkv + k])
          return fail(XQ_EINVAL, "XQ_DEBUG: the plan misses partition %d, kv head %d of sequence %d", sp, k, b);
  }
  return XQ_OK;
}

// length-aware plan: seq_tps[b] is a positive multiple of max(32, page_size) of at most
// kMaxSplitPages pages with ceil(context_lens[b] / seq_tps[b]) <= nsplits; every pair is {-1, *}
// or {unit, seq_tps[b]} of a unit of the launch, no unit appears twice, and every unit with
// tokens (and partition 0 of every sequence) appears.
xq_status debug_check_balanced(const xq_cache_layout* L, int32_t batch, int32_t nsplits, int32_t max_ctx,
                               const int32_t* context_lens, const int32_t* pairs, const int32_t* seq_tps,
                               hipStream_t s) {
  const int64_t hkv = L->num_kv_heads, units = (int64_t)nsplits * hkv * batch;
  const int32_t unit_tok = std::max<int32_t>(32, L->page_size);
  std::vector<int32_t> o, cl, tp;
  if (xq_status st = fetch(o, pairs, 2 * units, s)) return st;
  if (xq_status st = fetch(cl, context_lens, batch, s)) return st;
  if (xq_status st = fetch(tp, seq_tps, batch, s)) return st;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t Lb = std::min(std::max(cl[b], 0), max_ctx);
    if (tp[b] <= 0 || tp[b] % unit_tok != 0 || (int64_t)tp[b] > (int64_t)xq::kMaxSplitPages * L->page_size ||
        (Lb + tp[b] - 1) / tp[b] > nsplits)
      return fail(XQ_EINVAL, "XQ_DEBUG: seq_tps[%d] = %d is not a valid partition of %d tokens in %d", b, tp[b], Lb,
                  nsplits);
  }
  std::vector<char> seen((size_t)units, 0);
  for (int64_t i = 0; i < units; ++i) {
    const int32_t u = o[(size_t)(2 * i)];
    if (u == -1) continue;
    if (u < 0 || u >= units || seen[(size_t)u] || o[(size_t)(2 * i + 1)] != tp[(size_t)(u / hkv / nsplits)])
      return fail(XQ_EINVAL, "XQ_DEBUG: plan pair %lld = {%d, %d}: not -1 or a unit of the launch, once, with its "
                  "sequence's partition", (long long)i, u, o[(size_t)(2 * i + 1)]);
    seen[(size_t)u] = 1;
  }
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t Lb = std::min(std::max(cl[b], 0), max_ctx);
    const int32_t n = std::max(1, (Lb + tp[b] - 1) / tp[b]);
    for (int32_t sp = 0; sp < n; ++sp)
      for (int64_t k = 0; k < hkv; ++k)
        if (!seen[(size_t)(((int64_t)b * nsplits + sp) * hkv + k)])
          return fail(XQ_EINVAL, "XQ_DEBUG: the plan misses partition %d, kv head %lld of sequence %d", sp,
                      (long long)k, b);
  }
  return XQ_OK;
}

// prefill: the pages of positions 0 .. max_ctx - 1 in the chunk's block-table row are page ids
// in [0, num_pages).
xq_status debug_check_prefill(const xq_cache_layout* L, const int32_t* block_table, int32_t max_ctx,
                              hipStream_t s) {
  std::vector<int32_t> bt;
  const int32_t pages = (max_ctx + L->page_size - 1) / L->page_size;
  if (xq_status st = fetch(bt, block_table, pages, s)) return st;
  for (int32_t i = 0; i < pages; ++i)
    if (bt[i] < 0 || bt[i] >= L->num_pages)
      return fail(XQ_EINVAL, "XQ_DEBUG: block_table[%d] = %d is not a page id below num_pages = %lld", i, bt[i],
                  (long long)L->num_pages);
  return XQ_OK;
}

// append: token_seq >= 0, 0 <= token_pos < max_pages_per_seq * page_size, the page of every
// token is a page id in [0, num_pages), and no two tokens write the same (page, slot). The
// block table is read for rows 0 .. max(token_seq), the rows the kernel reads.
xq_status debug_check_append(const xq_cache_layout* L, int32_t n, const int32_t* token_seq,
                             const int32_t* token_pos, const int32_t* block_tables, int32_t maxp,
                             hipStream_t s) {
  std::vector<int32_t> seq, pos, bt;
  if (xq_status st = fetch(seq, token_seq, n, s)) return st;
  if (xq_status st = fetch(pos, token_pos, n, s)) return st;
  const int64_t cap = (int64_t)maxp * L->page_size;
  int32_t max_seq = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (seq[i] < 0) return fail(XQ_EINVAL, "XQ_DEBUG: token_seq[%d] = %d < 0", i, seq[i]);
    if (pos[i] < 0 || pos[i] >= cap)
      return fail(XQ_EINVAL, "XQ_DEBUG: token_pos[%d] = %d is outside [0, max_pages_per_seq * page_size = %lld)", i,
                  pos[i], (long long)cap);
    if (seq[i] > max_seq) max_seq = seq[i];
  }
  if (xq_status st = fetch(bt, block_tables, ((int64_t)max_seq + 1) * maxp, s)) return st;
  std::unordered_set<int64_t> slots;
  slots.reserve((size_t)n * 2);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pg = bt[(size_t)seq[i] * maxp + pos[i] / L->page_size];
    if (pg < 0 || pg >= L->num_pages)
      return fail(XQ_EINVAL, "XQ_DEBUG: token %d (sequence %d, position %d) maps to page %d, not below num_pages = %lld",
                  i, seq[i], pos[i], pg, (long long)L->num_pages);
    if (!slots.insert((int64_t)pg * L->page_size + pos[i] % L->page_size).second)
      return fail(XQ_EINVAL, "XQ_DEBUG: token %d writes page %d slot %d, already written by an earlier token", i, pg,
                  pos[i] % L->page_size);
  }
  return XQ_OK;
}

// rows appended by a decode launch beside its units: no row may land in a page that the decode
// reads (a page of sequences 0 .. batch - 1 holding one of their context_lens rows), since the
// launch's units and appenders run in no fixed order.
xq_status debug_check_disjoint(const xq_cache_layout* L, int32_t batch, const int32_t* context_lens,
                               const int32_t* block_tables, int32_t maxp, int32_t n, const int32_t* token_seq,
                               const int32_t* token_pos, hipStream_t s) {
  std::vector<int32_t> lens, seq, pos, bt;
  if (xq_status st = fetch(lens, context_lens, batch, s)) return st;
  if (xq_status st = fetch(seq, token_seq, n, s)) return st;
  if (xq_status st = fetch(pos, token_pos, n, s)) return st;
  int32_t rows = batch;
  for (int32_t i = 0; i < n; ++i) rows = std::max(rows, seq[i] + 1);
  if (xq_status st = fetch(bt, block_tables, (int64_t)rows * maxp, s)) return st;
  std::unordered_set<int32_t> read;
  for (int32_t b = 0; b < batch; ++b)
    for (int64_t t = 0; t < (int64_t)lens[b]; t += L->page_size) read.insert(bt[(size_t)b * maxp + t / L->page_size]);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pg = bt[(size_t)seq[i] * maxp + pos[i] / L->page_size];
    if (read.count(pg))
      return fail(XQ_EINVAL, "XQ_DEBUG: chunk row %d (sequence %d, position %d) writes page %d, which the decode reads",
                  i, seq[i], pos[i], pg);
  }
  return XQ_OK;
}

int64_t block_bytes_of(const xq_cache_layout* L) {
  const int64_t row = xq::row_code_bytes(L->kv_dtype);
  const int64_t bytes = L->page_size * row + (xq::has_scales(L->kv_dtype) ? 2 * L->page_size : 0);
  return (bytes + 15) & ~int64_t(15);
}

// A negative hint asks for fixed partitions of -hint tokens: whole pages, whole 32-token tiles and
// at most kMaxSplitPages pages.
bool fixed_split_ok(const xq_cache_layout* L, int32_t hint) {
  if (hint >= 0 || hint == INT32_MIN) return false;
  const int64_t tps = -(int64_t)hint, unit = L->page_size > 32 ? L->page_size : 32;
  return tps % unit == 0 && tps <= (int64_t)xq::kMaxSplitPages * L->page_size;
}

// Tokens per split: page aligned and a multiple of 32 (one tile of the decode kernel). hint > 0
// asks for that many splits of the longest sequence; 0 lets the library choose from the shape;
// hint < 0 (checked by fixed_split_ok) fixes the partition at -hint tokens.
int32_t plan_tokens_per_split(const xq_cache_layout* L, int32_t batch, int32_t max_ctx, int32_t hint) {
  if (hint < 0) return -hint;
  const int32_t ps = L->page_size;
  int64_t tps;
  if (hint > 0) {
    tps = (max_ctx + hint - 1) / hint;
  } else {
    // One wave per (split, kv head, sequence). Long splits amortise each wave's set-up and
    // epilogue; enough of them keep every compute unit busy: the longest power of two up to
    // 2048 tokens that still gives 4 waves per CU (8 for the dtypes that read tiles straight
    // into registers and rely on occupancy to hide latency), at least 64 tokens.
    const int64_t heads = (int64_t)batch * L->num_kv_heads;
    const int64_t target = (L->kv_dtype == 4 || L->kv_dtype == 8 || L->kv_dtype == 3) ? 1024 : 2048;
    tps = 2048;
    while (tps > 64 && heads * ((max_ctx + tps - 1) / tps) < target) tps >>= 1;
  }
  const int64_t unit = ps > 32 ? ps : 32;   // whole pages and whole 32-token tiles
  tps = ((tps + unit - 1) / unit) * unit;
  // a split spans at most kMaxSplitPages pages: the decode kernel keeps a split's block-table
  // entries in registers
  const int64_t cap = (int64_t)xq::kMaxSplitPages * ps;
  if (tps > cap) tps = cap;
  return (int32_t)tps;
}

// Shared by decode and prefill. Row b (a sequence, or a query token of a prefill chunk) reads
// block_tables + b * bt_stride and attends to context_lens[b] tokens (ctx_base == 0) or to
// ctx_base + b tokens (prefill: ctx_base = start_pos + 1, one shared table row).
xq_status attention(const xq_cache_layout* layout, const void* q, int32_t batch, int32_t num_q_heads,
                    const void* k_pool, const void* v_pool, const int32_t* block_tables, int32_t bt_stride,
                    int32_t max_pages_per_seq, const int32_t* context_lens, int32_t ctx_base,
                    int32_t max_context_len, float softmax_scale, int32_t num_splits_hint, void* workspace,
                    int64_t workspace_bytes, float* out, hipStream_t stream, const int32_t* seq_order = nullptr,
                    const void* k_new = nullptr, const void* v_new = nullptr, bool checked_ok = true,
                    const int32_t* seq_tps = nullptr, int32_t balanced_nsplits = 0,
                    const xq::AppendParams* extra = nullptr) {
  if (batch > 65535) return fail(XQ_EUNSUPPORTED, "batch %d > 65535", batch);
  if (num_q_heads < 1 || num_q_heads % layout->num_kv_heads != 0)
    return fail(XQ_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
                layout->num_kv_heads);
  const int32_t g = num_q_heads / layout->num_kv_heads;
  if (g > xq::kMaxGroup) return fail(XQ_EUNSUPPORTED, "group size %d > %d", g, xq::kMaxGroup);
  if (!q || !k_pool || !v_pool || !block_tables || !out)
    return fail(XQ_EINVAL, "a required pointer is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(XQ_EINVAL, "q, out and the pools must be 16-byte aligned");
  if (max_pages_per_seq < 1) return fail(XQ_EINVAL, "max_pages_per_seq %d < 1", max_pages_per_seq);
  if ((int64_t)max_context_len > (int64_t)max_pages_per_seq * layout->page_size)
    return fail(XQ_EINVAL, "context of %d tokens exceeds max_pages * page_size", max_context_len);
  if (num_splits_hint < 0 && !fixed_split_ok(layout, num_splits_hint))
    return fail(XQ_EINVAL,
                "num_splits_hint %d: a fixed partition must be a multiple of 32 tokens and of the page size, "
                "at most 128 pages", num_splits_hint);
  if (!(softmax_scale == softmax_scale)) return fail(XQ_EINVAL, "softmax_scale is NaN");

  const int32_t ctx = max_context_len > 0 ? max_context_len : 1;
  // a length-aware plan brings its own partitions (seq_tps) and their stride
  const int32_t tps = seq_tps ? 0 : plan_tokens_per_split(layout, batch, ctx, num_splits_hint);
  const int32_t nsplits = seq_tps ? balanced_nsplits : (ctx + tps - 1) / tps;
  if (nsplits > 65535) return fail(XQ_EUNSUPPORTED, "%d splits > 65535", nsplits);
  // One 64-lane workgroup per (split, kv head, row block) on a one-dimensional grid. A prefill
  // packs 16 / g query tokens (all g heads of each) into the 16 columns of a unit's MFMA tiles.
  const int32_t qt = ctx_base > 0 ? std::max(1, xq::kMaxGroup / g) : 1;
  const int64_t units = (int64_t)nsplits * layout->num_kv_heads * ((batch + qt - 1) / qt);
  if (units >= ((int64_t)1 << 26))
    return fail(XQ_EUNSUPPORTED, "%lld work units (splits x kv heads x rows) >= 2^26", (long long)units);
  if (extra && extra->n_tokens > 0 && checked_ok && debug_on())
    if (xq_status st = debug_check_append(layout, extra->n_tokens, extra->token_seq, extra->token_pos,
                                          extra->block_tables, extra->maxp, stream);
        st || (st = debug_check_disjoint(layout, batch, context_lens, block_tables, max_pages_per_seq,
                                         extra->n_tokens, extra->token_seq, extra->token_pos, stream)))
      return st;
  const xq::WorkspaceLayout ws = xq::workspace_layout(layout->kv_dtype, batch, num_q_heads, nsplits);
  if (ws.total > 0) {
    if (!workspace || workspace_bytes < ws.total)
      return fail(XQ_EWORKSPACE, "workspace of %lld bytes needed, %lld given", (long long)ws.total,
                  (long long)workspace_bytes);
    if (!aligned16(workspace)) return fail(XQ_EINVAL, "workspace must be 16-byte aligned");
  }
  uint8_t* wsp = static_cast<uint8_t*>(workspace);
  if (checked_ok && debug_on()) {
    xq_status st = ctx_base > 0 ? debug_check_prefill(layout, block_tables, max_context_len, stream)
                                : debug_check_decode(layout, batch, block_tables, max_pages_per_seq, context_lens,
                                                     max_context_len, stream);
    if (!st && seq_tps)
      st = debug_check_balanced(layout, batch, nsplits, max_context_len, context_lens, seq_order, seq_tps, stream);
    else if (!st && seq_order)
      st = nsplits > 1 ? debug_check_unit_plan(batch, layout->num_kv_heads, nsplits, tps, max_context_len, context_lens,
                                               seq_order, stream)
                       : debug_check_order(batch, seq_order, stream);
    if (st) return st;
  }

  xq::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k_pool = static_cast<const uint8_t*>(k_pool);
  p.v_pool = static_cast<const uint8_t*>(v_pool);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.partials = ws.part_bytes ? reinterpret_cast<float*>(wsp + ws.part_off) : nullptr;
  p.block_bytes = block_bytes_of(layout);
  p.page_stride = p.block_bytes * layout->num_kv_heads;
  p.pool_bytes = p.page_stride * layout->num_pages;
  p.batch = batch;
  p.hq = num_q_heads;
  p.hkv = layout->num_kv_heads;
  p.group = g;
  p.page_size = layout->page_size;
  p.page_shift = __builtin_ctz((unsigned)layout->page_size);
  p.maxp = max_pages_per_seq;
  p.tokens_per_split = tps;
  p.nsplits = nsplits;
  p.max_context_len = max_context_len;
  p.softmax_scale = softmax_scale;
  p.fixed_splits = num_splits_hint < 0 ? 1 : 0;
  p.bt_stride = bt_stride;
  p.ctx_base = ctx_base;
  p.qt = qt;
  p.seq_order = seq_order;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.seq_tps = seq_tps;
  if (extra && extra->n_tokens > 0) {
    // one pass = 16 rows; a workgroup per pass up to one per SIMD, looping beyond
    const int64_t passes = 2 * (((int64_t)extra->n_tokens + 15) / 16 * layout->num_kv_heads);
    p.xa = *extra;
    p.x_groups = (int32_t)std::min<int64_t>(passes, 1024);
  }
  const hipError_t e = xq::launch_decode(layout->kv_dtype, p, stream);
  if (e != hipSuccess) return fail(XQ_EHIP, "attention launch: %s", hipGetErrorString(e));
  return XQ_OK;
}

// ---- chunked prefill on the tile kernel ---------------------------------------------------
// Partitions of a tiled prefill: whole 64-token tiles and whole pages. hint > 0 asks for that many
// partitions of the longest query's context; 0 cuts the context only when the chunk's workgroups
// are fewer than two per compute unit, into partitions of at least 256 tokens (the query set-up and the partial store of a workgroup cost about as much as a few tiles).
struct TilePlan {
  int32_t tps, nsplits, block_queries;
};

TilePlan tile_prefill_plan(const xq_cache_layout* L, int32_t n_query, int32_t num_q_heads, int32_t ctx,
                           int32_t hint) {
  TilePlan t{};
  const int32_t g = num_q_heads / L->num_kv_heads;
  t.block_queries = xq::prefill_block_queries(g);
  const int64_t blocks = xq::prefill_workgroups(n_query, g, L->num_kv_heads, 1);
  const int64_t unit = L->page_size > 64 ? L->page_size : 64;
  int64_t tps;
  if (hint > 0) {
    tps = ((int64_t)ctx + hint - 1) / hint;
  } else {
    const int64_t want = blocks >= 512 ? 1 : (512 + blocks - 1) / blocks;
    tps = std::max<int64_t>(((int64_t)ctx + want - 1) / want, 256);
  }
  tps = (tps + unit - 1) / unit * unit;
  t.tps = (int32_t)std::min<int64_t>(tps, ((int64_t)ctx + unit - 1) / unit * unit);
  t.nsplits = (int32_t)(((int64_t)ctx + t.tps - 1) / t.tps);
  return t;
}

xq_status tile_prefill(const xq_cache_layout* layout, const void* q, int32_t n_query, int32_t num_q_heads,
                       const void* k_pool, const void* v_pool, const int32_t* block_table, int32_t max_pages,
                       int32_t start_pos, float softmax_scale, int32_t hint, void* workspace,
                       int64_t workspace_bytes, float* out, hipStream_t stream) {
  if (n_query > 65535) return fail(XQ_EUNSUPPORTED, "n_query %d > 65535", n_query);
  if (num_q_heads < 1 || num_q_heads % layout->num_kv_heads != 0)
    return fail(XQ_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
                layout->num_kv_heads);
  const int32_t g = num_q_heads / layout->num_kv_heads;
  if (g > xq::kMaxGroup) return fail(XQ_EUNSUPPORTED, "group size %d > %d", g, xq::kMaxGroup);
  if (!q || !k_pool || !v_pool || !block_table || !out) return fail(XQ_EINVAL, "a required pointer is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(XQ_EINVAL, "q, out and the pools must be 16-byte aligned");
  if (max_pages < 1) return fail(XQ_EINVAL, "max_pages %d < 1", max_pages);
  const int32_t ctx = start_pos + n_query;
  if ((int64_t)ctx > (int64_t)max_pages * layout->page_size)
    return fail(XQ_EINVAL, "context of %d tokens exceeds max_pages * page_size", ctx);
  if (!(softmax_scale == softmax_scale)) return fail(XQ_EINVAL, "softmax_scale is NaN");
  const TilePlan plan = tile_prefill_plan(layout, n_query, num_q_heads, ctx, hint);
  if (plan.nsplits > 65535) return fail(XQ_EUNSUPPORTED, "%d splits > 65535", plan.nsplits);
  const int64_t units = xq::prefill_workgroups(n_query, g, layout->num_kv_heads, plan.nsplits);
  if (units >= ((int64_t)1 << 31)) return fail(XQ_EUNSUPPORTED, "%lld workgroups", (long long)units);
  const xq::WorkspaceLayout ws = xq::workspace_layout(layout->kv_dtype, n_query, num_q_heads, plan.nsplits);
  if (ws.total > 0) {
    if (!workspace || workspace_bytes < ws.total)
      return fail(XQ_EWORKSPACE, "workspace of %lld bytes needed (xq_prefill_workspace_bytes), %lld given",
                  (long long)ws.total, (long long)workspace_bytes);
    if (!aligned16(workspace)) return fail(XQ_EINVAL, "workspace must be 16-byte aligned");
  }
  if (debug_on())
    if (xq_status st = debug_check_prefill(layout, block_table, ctx, stream)) return st;

  xq::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k_pool = static_cast<const uint8_t*>(k_pool);
  p.v_pool = static_cast<const uint8_t*>(v_pool);
  p.block_tables = block_table;
  p.out = out;
  p.partials = ws.part_bytes ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ws.part_off) : nullptr;
  p.block_bytes = block_bytes_of(layout);
  p.page_stride = p.block_bytes * layout->num_kv_heads;
  p.pool_bytes = p.page_stride * layout->num_pages;
  p.batch = n_query;
  p.hq = num_q_heads;
  p.hkv = layout->num_kv_heads;
  p.group = g;
  p.page_size = layout->page_size;
  p.page_shift = __builtin_ctz((unsigned)layout->page_size);
  p.maxp = max_pages;
  p.tokens_per_split = plan.tps;
  p.nsplits = plan.nsplits;
  p.max_context_len = ctx;
  p.softmax_scale = softmax_scale;
  p.ctx_base = start_pos + 1;
  p.qt = plan.block_queries;
  const hipError_t e = xq::launch_prefill(layout->kv_dtype, p, stream);
  if (e != hipSuccess) return fail(XQ_EHIP, "prefill launch: %s", hipGetErrorString(e));
  return XQ_OK;
}

// ---- scratch of the allocation-free decode ----------------------------------------------
// xq_paged_decode_attention_noalloc keeps its split partials in this file-scope device array: one
// copy per GPU the library runs on, held until the process ends. In host code `scratch` is only
// a stand-in for the symbol; its device address on each device comes from hipGetSymbolAddress,
// taken once per device (with that device current) on the entry point's first call there.
constexpr int64_t kScratchBytes = int64_t(16) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// A plan's entry count must be the one xq_decode_plan writes for these arguments: the kernel reads
// one entry per sequence or per work slot and cannot check the array's length.
xq_status check_plan_entries(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                             int32_t max_context_len, int32_t num_splits_hint, int32_t plan_entries);

xq_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(XQ_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(XQ_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(XQ_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return XQ_OK;
}

}  // namespace

extern "C" {

int64_t xq_block_bytes(const xq_cache_layout* layout) {
  if (check_layout(layout) != XQ_OK) return -1;
  return block_bytes_of(layout);
}

int64_t xq_page_stride_bytes(const xq_cache_layout* layout) {
  if (check_layout(layout) != XQ_OK) return -1;
  return block_bytes_of(layout) * layout->num_kv_heads;
}

int64_t xq_pool_bytes(const xq_cache_layout* layout) {
  if (check_layout(layout) != XQ_OK) return -1;
  return block_bytes_of(layout) * layout->num_kv_heads * layout->num_pages;
}

int32_t xq_decode_num_splits(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                             int32_t max_context_len, int32_t num_splits_hint) {
  if (check_layout(layout) != XQ_OK) return -1;
  if (batch < 0 || num_q_heads < 1 || max_context_len < 0) return -1;
  if (num_splits_hint < 0 && !fixed_split_ok(layout, num_splits_hint)) return -1;
  if (max_context_len == 0) return 1;
  const int32_t tps = plan_tokens_per_split(layout, batch, max_context_len, num_splits_hint);
  return (max_context_len + tps - 1) / tps;
}

int64_t xq_decode_workspace_bytes(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t num_splits_hint) {
  const int32_t ns = xq_decode_num_splits(layout, batch, num_q_heads, max_context_len, num_splits_hint);
  if (ns < 0) return -1;
  return xq::workspace_layout(layout->kv_dtype, batch, num_q_heads, ns).total;
}

const char* xq_status_string(int32_t status) {
  switch (status) {
    case XQ_OK: return "ok";
    case XQ_EINVAL: return "invalid argument";
    case XQ_EUNSUPPORTED: return "unsupported configuration";
    case XQ_EWORKSPACE: return "workspace too small";
    case XQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* xq_last_error(void) { return g_last_error.c_str(); }

xq_status xq_quantize_append(const xq_cache_layout* layout, const void* k_new, const void* v_new,
                             int32_t n_tokens, const int32_t* token_seq, const int32_t* token_pos,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             void* k_pool, void* v_pool, void* stream) {
  if (xq_status st = check_layout(layout)) return st;
  if (n_tokens < 0) return fail(XQ_EINVAL, "n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) return XQ_OK;
  if (!k_new || !v_new || !token_seq || !token_pos || !block_tables || !k_pool || !v_pool)
    return fail(XQ_EINVAL, "a required pointer is NULL");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(XQ_EINVAL, "k_new, v_new and the pools must be 16-byte aligned");
  if (max_pages_per_seq < 1) return fail(XQ_EINVAL, "max_pages_per_seq %d < 1", max_pages_per_seq);
  // one 16-lane group per (token, kv head) row: the launch's work-items (16 per row) must stay
  // below 2^32
  if ((int64_t)n_tokens * layout->num_kv_heads >= ((int64_t)1 << 28))
    return fail(XQ_EUNSUPPORTED, "n_tokens * num_kv_heads = %lld rows: at most 2^28 - 1 per call",
                (long long)n_tokens * layout->num_kv_heads);
  if (debug_on())
    if (xq_status st = debug_check_append(layout, n_tokens, token_seq, token_pos, block_tables, max_pages_per_seq,
                                          static_cast<hipStream_t>(stream)))
      return st;
  xq::AppendParams p{};
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.token_seq = token_seq;
  p.token_pos = token_pos;
  p.block_tables = block_tables;
  p.k_pool = static_cast<uint8_t*>(k_pool);
  p.v_pool = static_cast<uint8_t*>(v_pool);
  p.block_bytes = block_bytes_of(layout);
  p.page_stride = p.block_bytes * layout->num_kv_heads;
  p.n_tokens = n_tokens;
  p.hkv = layout->num_kv_heads;
  p.page_size = layout->page_size;
  p.maxp = max_pages_per_seq;
  const hipError_t e = xq::launch_quantize_append(layout->kv_dtype, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(XQ_EHIP, "quantize_append launch: %s", hipGetErrorString(e));
  return XQ_OK;
}

xq_status xq_paged_decode_attention(const xq_cache_layout* layout, const void* q, int32_t batch,
                                    int32_t num_q_heads, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, int32_t max_pages_per_seq,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    float softmax_scale, int32_t num_splits_hint, void* workspace,
                                    int64_t workspace_bytes, float* out, void* stream) {
  if (xq_status st = check_layout(layout)) return st;
  if (batch < 0) return fail(XQ_EINVAL, "batch %d < 0", batch);
  if (batch == 0) return XQ_OK;
  if (!context_lens) return fail(XQ_EINVAL, "a required pointer is NULL");
  if (max_context_len < 0) return fail(XQ_EINVAL, "max_context_len %d < 0", max_context_len);
  return attention(layout, q, batch, num_q_heads, k_pool, v_pool, block_tables, max_pages_per_seq,
                   max_pages_per_seq, context_lens, 0, max_context_len, softmax_scale, num_splits_hint,
                   workspace, workspace_bytes, out, static_cast<hipStream_t>(stream));
}

xq_status xq_paged_decode_attention_noalloc(const xq_cache_layout* layout, const void* q, int32_t batch,
                                            int32_t num_q_heads, const void* k_pool, const void* v_pool,
                                            const int32_t* block_tables, int32_t max_pages_per_seq,
                                            const int32_t* context_lens, int32_t max_context_len,
                                            float softmax_scale, int32_t num_splits_hint, float* out,
                                            void* stream) {
  if (xq_status st = check_layout(layout)) return st;
  if (batch < 0) return fail(XQ_EINVAL, "batch %d < 0", batch);
  if (batch == 0) return XQ_OK;
  if (!context_lens) return fail(XQ_EINVAL, "a required pointer is NULL");
  if (max_context_len < 0) return fail(XQ_EINVAL, "max_context_len %d < 0", max_context_len);
  const int64_t need = xq_decode_workspace_bytes(layout, batch, num_q_heads, max_context_len, num_splits_hint);
  if (need < 0) return fail(XQ_EINVAL, "invalid batch, head count, context length or split hint");
  if (need > kScratchBytes)
    return fail(XQ_EWORKSPACE, "split partials of %lld bytes needed; the built-in scratch holds %lld",
                (long long)need, (long long)kScratchBytes);
  void* ws = nullptr;
  if (xq_status st = scratch_address(&ws)) return st;
  return attention(layout, q, batch, num_q_heads, k_pool, v_pool, block_tables, max_pages_per_seq,
                   max_pages_per_seq, context_lens, 0, max_context_len, softmax_scale, num_splits_hint, ws,
                   kScratchBytes, out, static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr, false);
}

xq_status xq_paged_decode_attention_planned(const xq_cache_layout* layout, const void* q, int32_t batch,
                                            int32_t num_q_heads, const void* k_pool, const void* v_pool,
                                            const int32_t* block_tables, int32_t max_pages_per_seq,
                                            const int32_t* context_lens, int32_t max_context_len,
                                            float softmax_scale, int32_t num_splits_hint, void* workspace,
                                            int64_t workspace_bytes, float* out, const int32_t* seq_order,
                                            int32_t plan_entries, void* stream) {
  if (xq_status st = check_layout(layout)) return st;
  if (batch < 0) return fail(XQ_EINVAL, "batch %d < 0", batch);
  if (batch == 0) return XQ_OK;
  if (!context_lens || !seq_order) return fail(XQ_EINVAL, "a required pointer is NULL");
  if (max_context_len < 0) return fail(XQ_EINVAL, "max_context_len %d < 0", max_context_len);
  if (xq_status st = check_plan_entries(layout, batch, num_q_heads, max_context_len, num_splits_hint, plan_entries))
    return st;
  return attention(layout, q, batch, num_q_heads, k_pool, v_pool, block_tables, max_pages_per_seq,
                   max_pages_per_seq, context_lens, 0, max_context_len, softmax_scale, num_splits_hint,
                   workspace, workspace_bytes, out, static_cast<hipStream_t>(stream), seq_order);
}

xq_status xq_append_decode_attention(const xq_cache_layout* layout, const void* k_new, const void* v_new,
                                     const void* q, int32_t batch, int32_t num_q_heads, void* k_pool,
                                     void* v_pool, const int32_t* block_tables, int32_t max_pages_per_seq,
                                     const int32_t* context_lens, int32_t max_context_len, float softmax_scale,
                                     int32_t num_splits_hint, void* workspace, int64_t workspace_bytes,
                                     float* out, const int32_t* seq_order, int32_t plan_entries, void* stream) {
  if (xq_status st = check_layout(layout)) return st;
  if (batch < 0) return fail(XQ_EINVAL, "batch %d < 0", batch);
  if (batch == 0) return XQ_OK;
  if (!context_lens || !k_new || !v_new) return fail(XQ_EINVAL, "a required pointer is NULL");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(XQ_EINVAL, "k_new and v_new must be 16-byte aligned");
  if (max_context_len < 0) return fail(XQ_EINVAL, "max_context_len %d < 0", max_context_len);
  if (seq_order)
    if (xq_status st = check_plan_entries(layout, batch, num_q_heads, max_context_len, num_splits_hint, plan_entries))
      return st;
  return attention(layout, q, batch, num_q_heads, k_pool, v_pool, block_tables, max_pages_per_seq,
                   max_pages_per_seq, context_lens, 0, max_context_len, softmax_scale, num_splits_hint,
                   workspace, workspace_bytes, out, static_cast<hipStream_t>(stream), seq_order, k_new, v_new);
}

int32_t xq_decode_plan_entries(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                               int32_t max_context_len, int32_t num_splits_hint) {
  if (check_layout(layout) != XQ_OK) return -1;
  if (batch < 0 || num_q_heads < 1 || max_context_len < 0) return -1;
  if (num_splits_hint < 0 && !fixed_split_ok(layout, num_splits_hint)) return -1;
  if (batch == 0) return 0;
  const int32_t ctx = max_context_len > 0 ? max_context_len : 1;
  const int32_t tps = plan_tokens_per_split(layout, batch, ctx, num_splits_hint);
  const int64_t nsplits = (ctx + tps - 1) / tps;
  if (nsplits == 1) return batch;
  const int64_t units = nsplits * layout->num_kv_heads * batch;
  return units >= ((int64_t)1 << 26) ? -1 : (int32_t)units;
}

xq_status xq_decode_plan(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                         int32_t max_context_len, int32_t num_splits_hint, const int32_t* host_context_lens,
                         int32_t* host_seq_order) {
  if (xq_status st = check_layout(layout)) return st;
  if (batch < 0 || num_q_heads < 1 || max_context_len < 0) return fail(XQ_EINVAL, "invalid batch, heads or length");
  if (batch > 0 && (!host_context_lens || !host_seq_order)) return fail(XQ_EINVAL, "a required pointer is NULL");
  if (num_splits_hint < 0 && !fixed_split_ok(layout, num_splits_hint))
    return fail(XQ_EINVAL, "num_splits_hint %d is not a valid fixed partition", num_splits_hint);
  if (batch == 0) return XQ_OK;
  const int32_t ctx = max_context_len > 0 ? max_context_len : 1;
  const int32_t tps = plan_tokens_per_split(layout, batch, ctx, num_splits_hint);
  const int32_t nsplits = (ctx + tps - 1) / tps;
  const int64_t hkv = layout->num_kv_heads;
  int simds = 1024;   // MI355X: 256 compute units x 4 SIMDs, if the device cannot be asked
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    simds = 4 * cus;
  else
    (void)hipGetLastError();

  if (nsplits == 1) {
    // Waves fill the SIMDs round-robin: with every unit resident, workgroups i, i + S, i + 2S, ...
    // (S = SIMDs of the device) share a SIMD. With one partition per sequence and a batch that is
    // a multiple of 8, the decode's unit order puts sequence slots b, b + S / Hkv, b + 2 S / Hkv,
    // ... on the same SIMDs (all their kv heads). Sorted by length, sequences are dealt to those
    // slot groups in snake order, so a SIMD's units add up to about the same number of tiles.
    for (int32_t b = 0; b < batch; ++b) host_seq_order[b] = b;
    if (batch % 8 != 0 || simds % (8 * hkv) != 0) return XQ_OK;
    const int64_t period = simds / hkv;   // slots b and b + period share SIMDs
    if (period >= batch) return XQ_OK;
    std::vector<int32_t> idx((size_t)batch);
    for (int32_t b = 0; b < batch; ++b) idx[(size_t)b] = b;
    std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) {
      return host_context_lens[a] > host_context_lens[b];
    });
    size_t next = 0;
    for (int64_t k = 0; next < idx.size(); ++k) {       // pass k fills member k of every group
      for (int64_t j = 0; j < period && next < idx.size(); ++j) {
        const int64_t group = (k & 1) ? period - 1 - j : j;
        const int64_t slot = group + k * period;
        if (slot < batch) host_seq_order[slot] = idx[next++];
      }
    }
    return XQ_OK;
  }

  // Several partitions: a unit plan, one entry per work slot (workgroup id) of the launch, giving
  // the unit (b nsplits + split) hkv + kvh it runs or -1. The n units with work come first, in ids
  // 0 .. n-1, and every later id is -1: a workgroup that exits at once frees its slot for the next
  // id, so a -1 among the first ids would move every later workgroup off its SIMD. With the first
  // ids resident (R waves per SIMD), workgroup i runs on SIMD i mod S. The (sequence, partition)
  // groups, each hkv units of equal length, are placed longest first (LPT) on the least loaded
  // column of SIMDs that has a free cell, a group's kv heads on one XCD (XCD = id mod 8) so that
  // its L2 fetches each line of a page once: the cell of column (x, y) in round r holds ids
  // x + 8 (hkv y + k) + S r, k < hkv, and is free when all of them are below min(n, R S).
  // Groups left over fill the ids below n that no cell took, then the ones after, in the same
  // longest-first order.
  const int64_t units = (int64_t)nsplits * hkv * batch;
  if (units >= ((int64_t)1 << 26)) return fail(XQ_EUNSUPPORTED, "%lld work units >= 2^26", (long long)units);
  for (int64_t i = 0; i < units; ++i) host_seq_order[i] = -1;
  struct Group { int32_t b, split, tiles; };
  std::vector<Group> groups;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t L = std::min(std::max(host_context_lens[b], 0), max_context_len);
    // partition 0 of an empty sequence too: its unit writes the sequence's zero output
    for (int32_t sp = 0; sp == 0 || (int64_t)sp * tps < L; ++sp) {
      const int32_t n = std::max(0, std::min(L, (sp + 1) * tps) - sp * tps);
      groups.push_back({b, sp, (n + 31) / 32});
    }
  }
  std::stable_sort(groups.begin(), groups.end(), [](const Group& a, const Group& c) { return a.tiles > c.tiles; });
  auto unit = [&](const Group& g, int64_t k) { return (int32_t)(((int64_t)g.b * nsplits + g.split) * hkv + k); };
  const int64_t n = (int64_t)groups.size() * hkv;   // units with work, ids 0 .. n-1
  xq::DecodeParams q{};
  q.batch = batch;
  q.hkv = (int32_t)hkv;
  q.nsplits = nsplits;
  q.qt = 1;
  q.fixed_splits = num_splits_hint < 0 ? 1 : 0;
  // columns of hkv SIMDs in one XCD; without them (a SIMD count that is not a multiple of 8 hkv) no
  // placement, only the longest-first order
  const int64_t cols = (simds % (8 * hkv) == 0) ? simds / hkv : 0;
  const int64_t rounds = cols > 0 ? xq::decode_waves_per_simd(layout->kv_dtype, q) : 0;
  const int64_t limit = std::min<int64_t>(n, rounds * simds);   // cells lie below this id
  std::vector<int64_t> load((size_t)cols, 0), used((size_t)cols, 0), cap((size_t)cols, 0);
  for (int64_t c = 0; c < cols; ++c)
    for (int64_t r = 0; r < rounds; ++r)
      if (c % 8 + 8 * (hkv * (c / 8) + hkv - 1) + simds * r < limit) cap[(size_t)c] = r + 1;
  std::vector<const Group*> rest;
  for (const Group& g : groups) {
    int64_t best = -1;
    for (int64_t c = 0; c < cols; ++c)
      if (used[(size_t)c] < cap[(size_t)c] && (best < 0 || load[(size_t)c] < load[(size_t)best])) best = c;
    if (best >= 0) {
      const int64_t x = best % 8, y = best / 8, r = used[(size_t)best]++;
      load[(size_t)best] += g.tiles;
      for (int64_t k = 0; k < hkv; ++k) host_seq_order[x + 8 * (hkv * y + k) + simds * r] = unit(g, k);
    } else {
      rest.push_back(&g);
    }
  }
  int64_t next = 0;
  for (const Group* g : rest)
    for (int64_t k = 0; k < hkv; ++k) {
      while (host_seq_order[next] >= 0) ++next;   // the next id no cell took (below n first)
      host_seq_order[next++] = unit(*g, k);
    }
  return XQ_OK;
}

int32_t xq_decode_plan_balanced(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                                int32_t max_context_len, const int32_t* host_context_lens, int32_t* host_seq_tps,
                                int32_t* host_units) {
  if (check_layout(layout) != XQ_OK) return -1;
  if (batch < 0 || num_q_heads < 1 || num_q_heads % layout->num_kv_heads != 0 || max_context_len < 0) {
    fail(XQ_EINVAL, "invalid batch, head count or context length");
    return -1;
  }
  if (batch == 0) return 1;
  if (!host_context_lens || !host_seq_tps) {
    fail(XQ_EINVAL, "a required pointer is NULL");
    return -1;
  }
  const int64_t hkv = layout->num_kv_heads;
  const int32_t ps = layout->page_size;
  const int32_t unit_tok = std::max<int32_t>(32, ps), unit_tiles = unit_tok / 32;   // whole tiles and pages
  const int32_t cap_tiles = xq::kMaxSplitPages * ps / 32;                           // the block-table window
  int simds = 1024;   // MI355X: 256 compute units x 4 SIMDs, if the device cannot be asked
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    simds = 4 * cus;
  else
    (void)hipGetLastError();

  // Partitions of about T tiles each, T the smallest (in whole pages) for which all units fit the
  // waves resident at once: every SIMD then runs the same number of units of about the same length,
  // whatever SIMD of its compute unit the hardware gives each of them. T is at least 32 tiles
  // (1,024 tokens) where partitions that long still give half the resident waves work: below
  // that a unit's set-up, partials and merge cost more than the balance gains (measured on
  // MI355X, 256 sequences of 64 to 1,024 tokens: 42.3 us unsplit, 45.8 us in partitions of 12
  // tiles; 64 sequences of 1,024 to 32,768 tokens: 130 us in partitions of about 48 tiles, 139 us
  // in uniform ones of 64 tiles). A small batch keeps short partitions: its units run alone, and
  // more of them shorten the longest.
  std::vector<int32_t> Lb((size_t)batch), tiles((size_t)batch);
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    Lb[(size_t)b] = std::min(std::max(host_context_lens[b], 0), max_context_len);
    tiles[(size_t)b] = (Lb[(size_t)b] + 31) / 32;
    total += tiles[(size_t)b] * hkv;
  }
  auto units_for = [&](int64_t T) {
    int64_t n = 0;
    for (int32_t b = 0; b < batch; ++b) n += std::max<int64_t>(1, (tiles[(size_t)b] + T - 1) / T) * hkv;
    return n;
  };
  auto tiles_per_unit = [&](int64_t slots) {
    int64_t T = std::max<int64_t>(unit_tiles, (total + slots - 1) / slots);
    if (T < 32 && units_for(32) >= slots / 2) T = 32;
    T = (T + unit_tiles - 1) / unit_tiles * unit_tiles;
    while (T < cap_tiles && units_for(T) > slots) T += unit_tiles;
    return std::min<int64_t>(T, cap_tiles);
  };
  auto stride_for = [&](int64_t T) {
    int32_t ns = 1;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t parts = std::max<int64_t>(1, (tiles[(size_t)b] + T - 1) / T);
      int64_t tps = (Lb[(size_t)b] + parts - 1) / parts;
      tps = std::min<int64_t>(std::max<int64_t>(unit_tok, (tps + unit_tok - 1) / unit_tok * unit_tok),
                              (int64_t)cap_tiles * 32);
      host_seq_tps[b] = (int32_t)tps;
      ns = std::max<int32_t>(ns, (int32_t)std::max<int64_t>(1, (Lb[(size_t)b] + tps - 1) / tps));
    }
    return ns;
  };
  // resident waves per SIMD of the launch (its ring depth follows its unit count): estimated for a
  // launch of many units, then taken again for the stride found
  xq::DecodeParams q{};
  q.batch = batch;
  q.hkv = (int32_t)hkv;
  q.qt = 1;
  q.nsplits = (int32_t)std::max<int64_t>(1, (3 * (int64_t)simds + batch * hkv - 1) / (batch * hkv));
  int64_t R = xq::decode_waves_per_simd(layout->kv_dtype, q);
  int32_t nsplits = stride_for(tiles_per_unit(R * simds));
  q.nsplits = nsplits;
  const int64_t R2 = xq::decode_waves_per_simd(layout->kv_dtype, q);
  if (R2 != R) {
    R = R2;
    nsplits = stride_for(tiles_per_unit(R * simds));
  }
  if ((int64_t)nsplits * hkv * batch >= ((int64_t)1 << 26)) {
    fail(XQ_EUNSUPPORTED, "%lld work units >= 2^26", (long long)nsplits * hkv * batch);
    return -1;
  }
  if (!host_units) return nsplits;

  // The units, longest first, in ids 0 .. n-1 (later ids: {-1, 0}); workgroup i runs on XCD
  // i mod 8 and compute unit i mod C (C = SIMDs / 4), and, while the first ids are all resident
  // (measured: with two waves per SIMD), on SIMD i mod S. Whole rounds of S ids deal the
  // (sequence, partition) groups to columns of hkv SIMDs in one XCD, snaking, so that the units
  // sharing a SIMD (and a compute unit) sum to about the same; the column (x, y) of round r holds
  // ids x + 8 (hkv y + k) + S r, k < hkv, so a group's kv heads share an XCD's L2. The groups
  // after the whole rounds follow in order.
  const int64_t entries = (int64_t)nsplits * hkv * batch;
  for (int64_t i = 0; i < entries; ++i) {
    host_units[2 * i] = -1;
    host_units[2 * i + 1] = 0;
  }
  struct Group { int32_t b, split, tiles; };
  std::vector<Group> groups;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t tps = host_seq_tps[b];
    for (int32_t sp = 0; sp == 0 || (int64_t)sp * tps < Lb[(size_t)b]; ++sp) {
      const int32_t n = std::max(0, std::min(Lb[(size_t)b], (sp + 1) * tps) - sp * tps);
      groups.push_back({b, sp, (n + 31) / 32});
    }
  }
  std::stable_sort(groups.begin(), groups.end(), [](const Group& a, const Group& c) { return a.tiles > c.tiles; });
  const int64_t C = simds;   // ids per round
  const int64_t cols = (C % (8 * hkv) == 0) ? C / hkv : 0;
  const int64_t full = cols > 0 ? (int64_t)groups.size() / cols : 0;   // whole rounds
  for (int64_t gi = 0; gi < (int64_t)groups.size(); ++gi) {
    const Group& g = groups[(size_t)gi];
    const int32_t u0 = (int32_t)(((int64_t)g.b * nsplits + g.split) * hkv);
    for (int64_t k = 0; k < hkv; ++k) {
      int64_t id;
      const int64_t r = cols > 0 ? gi / cols : 0;
      if (r < full) {
        int64_t j = gi % cols;
        if (r & 1) j = cols - 1 - j;
        id = j % 8 + 8 * (hkv * (j / 8) + k) + C * r;
      } else {
        id = full * cols * hkv + (gi - full * cols) * hkv + k;
      }
      host_units[2 * id] = u0 + (int32_t)k;
      host_units[2 * id + 1] = host_seq_tps[g.b];
    }
  }
  return nsplits;
}

int64_t xq_decode_workspace_bytes_balanced(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                                           int32_t nsplits) {
  if (check_layout(layout) != XQ_OK) return -1;
  if (batch < 0 || num_q_heads < 1 || nsplits < 1) return -1;
  return xq::workspace_layout(layout->kv_dtype, batch, num_q_heads, nsplits).total;
}

xq_status xq_decode_attention_balanced(const xq_cache_layout* layout, const void* q, int32_t batch,
                                       int32_t num_q_heads, void* k_pool, void* v_pool,
                                       const int32_t* block_tables, int32_t max_pages_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len, float softmax_scale,
                                       int32_t nsplits, const int32_t* units, const int32_t* seq_tps,
                                       const void* k_new, const void* v_new, const void* chunk_k,
                                       const void* chunk_v, int32_t chunk_tokens, const int32_t* chunk_seq,
                                       const int32_t* chunk_pos, void* workspace, int64_t workspace_bytes,
                                       float* out, void* stream) {
  if (xq_status st = check_layout(layout)) return st;
  if (batch < 0) return fail(XQ_EINVAL, "batch %d < 0", batch);
  if (batch == 0) return XQ_OK;
  if (!context_lens || !units || !seq_tps) return fail(XQ_EINVAL, "a required pointer is NULL");
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(XQ_EINVAL, "k_new and v_new: both or neither");
  if (k_new && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(XQ_EINVAL, "k_new and v_new must be 16-byte aligned");
  if (nsplits < 1) return fail(XQ_EINVAL, "nsplits %d < 1", nsplits);
  if (max_context_len < 0) return fail(XQ_EINVAL, "max_context_len %d < 0", max_context_len);
  if (chunk_tokens < 0) return fail(XQ_EINVAL, "chunk_tokens %d < 0", chunk_tokens);
  xq::AppendParams x{};
  if (chunk_tokens > 0) {
    if (!chunk_k || !chunk_v || !chunk_seq || !chunk_pos) return fail(XQ_EINVAL, "a required chunk pointer is NULL");
    if (!aligned16(chunk_k) || !aligned16(chunk_v)) return fail(XQ_EINVAL, "chunk_k and chunk_v must be 16-byte aligned");
    if ((int64_t)chunk_tokens * layout->num_kv_heads >= ((int64_t)1 << 28))
      return fail(XQ_EUNSUPPORTED, "chunk_tokens * num_kv_heads = %lld rows: at most 2^28 - 1 per call",
                  (long long)chunk_tokens * layout->num_kv_heads);
    x.k_new = static_cast<const uint16_t*>(chunk_k);
    x.v_new = static_cast<const uint16_t*>(chunk_v);
    x.token_seq = chunk_seq;
    x.token_pos = chunk_pos;
    x.block_tables = block_tables;
    x.k_pool = static_cast<uint8_t*>(k_pool);
    x.v_pool = static_cast<uint8_t*>(v_pool);
    x.block_bytes = block_bytes_of(layout);
    x.page_stride = x.block_bytes * layout->num_kv_heads;
    x.n_tokens = chunk_tokens;
    x.hkv = layout->num_kv_heads;
    x.page_size = layout->page_size;
    x.maxp = max_pages_per_seq;
  }
  return attention(layout, q, batch, num_q_heads, k_pool, v_pool, block_tables, max_pages_per_seq,
                   max_pages_per_seq, context_lens, 0, max_context_len, softmax_scale, 0, workspace,
                   workspace_bytes, out, static_cast<hipStream_t>(stream), units, k_new, v_new, true, seq_tps,
                   nsplits, &x);
}

int64_t xq_prefill_workspace_bytes(const xq_cache_layout* layout, int32_t n_query, int32_t num_q_heads,
                                   int32_t start_pos, int32_t num_splits_hint) {
  if (check_layout(layout) || n_query < 0 || start_pos < 0 || num_q_heads < 1 ||
      num_q_heads % layout->num_kv_heads != 0 || num_q_heads / layout->num_kv_heads > xq::kMaxGroup ||
      (int64_t)start_pos + n_query > INT32_MAX / 2)
    return -1;
  if (n_query == 0) return 0;
  if (num_splits_hint < 0 || !xq::prefill_tiled(layout->kv_dtype))
    return xq_decode_workspace_bytes(layout, n_query, num_q_heads, start_pos + n_query, num_splits_hint);
  const int32_t ns = tile_prefill_plan(layout, n_query, num_q_heads, start_pos + n_query, num_splits_hint).nsplits;
  return xq::workspace_layout(layout->kv_dtype, n_query, num_q_heads, ns).total;
}

xq_status xq_paged_prefill_attention(const xq_cache_layout* layout, const void* q, int32_t n_query,
                                     int32_t num_q_heads, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, int32_t max_pages, int32_t start_pos,
                                     float softmax_scale, int32_t num_splits_hint, void* workspace,
                                     int64_t workspace_bytes, float* out, void* stream) {
  if (xq_status st = check_layout(layout)) return st;
  if (n_query < 0) return fail(XQ_EINVAL, "n_query %d < 0", n_query);
  if (start_pos < 0) return fail(XQ_EINVAL, "start_pos %d < 0", start_pos);
  if (n_query == 0) return XQ_OK;
  if ((int64_t)start_pos + n_query > INT32_MAX / 2)
    return fail(XQ_EINVAL, "start_pos + n_query = %lld is too large", (long long)start_pos + n_query);
  if (num_splits_hint >= 0 && xq::prefill_tiled(layout->kv_dtype))
    return tile_prefill(layout, q, n_query, num_q_heads, k_pool, v_pool, block_table, max_pages, start_pos,
                        softmax_scale, num_splits_hint, workspace, workspace_bytes, out,
                        static_cast<hipStream_t>(stream));
  return attention(layout, q, n_query, num_q_heads, k_pool, v_pool, block_table, 0, max_pages, nullptr,
                   start_pos + 1, start_pos + n_query, softmax_scale, num_splits_hint, workspace,
                   workspace_bytes, out, static_cast<hipStream_t>(stream));
}

xq_status xq_hbm_read_probe(const void* buf, int64_t buf_bytes, int64_t n_blocks, int32_t block_bytes,
                             int64_t block_stride, const int32_t* block_order, uint32_t* sink, void* stream) {
  if (n_blocks < 0) return fail(XQ_EINVAL, "n_blocks %lld < 0", (long long)n_blocks);
  if (n_blocks == 0) return XQ_OK;
  if (!buf || !sink) return fail(XQ_EINVAL, "a required pointer is NULL");
  if (!aligned16(buf)) return fail(XQ_EINVAL, "buf must be 16-byte aligned");
  if (block_bytes < 1024 || block_bytes > (1 << 20) || !pow2(block_bytes))
    return fail(XQ_EINVAL, "block_bytes %d is not a power of two in [1024, 2^20]", block_bytes);
  if (block_stride < block_bytes || block_stride % 16 != 0)
    return fail(XQ_EINVAL, "block_stride %lld must be a multiple of 16 and at least block_bytes",
                (long long)block_stride);
  if (n_blocks * (block_bytes / 1024) > INT32_MAX)
    return fail(XQ_EUNSUPPORTED, "n_blocks * block_bytes is 2 TiB or more", (long long)n_blocks);
  if (!block_order && (n_blocks - 1) * block_stride + block_bytes > buf_bytes)
    return fail(XQ_EINVAL, "n_blocks blocks at block_stride do not fit buf_bytes");
  const hipError_t e = xq::launch_hbm_probe(static_cast<const uint8_t*>(buf), n_blocks, block_bytes, block_stride,
                                            block_order, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(XQ_EHIP, "hbm probe launch: %s", hipGetErrorString(e));
  return XQ_OK;
}

}  // extern "C"

namespace {
xq_status check_plan_entries(const xq_cache_layout* layout, int32_t batch, int32_t num_q_heads,
                             int32_t max_context_len, int32_t num_splits_hint, int32_t plan_entries) {
  const int32_t want = xq_decode_plan_entries(layout, batch, num_q_heads, max_context_len, num_splits_hint);
  if (want < 0) return fail(XQ_EINVAL, "invalid batch, head count, context length or split hint");
  if (plan_entries != want)
    return fail(XQ_EINVAL, "plan of %d entries given; these arguments take a plan of %d (xq_decode_plan_entries)",
                plan_entries, want);
  return XQ_OK;
}
}  // namespace
