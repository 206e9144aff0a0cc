// Host side of libpagedattn: argument checks, workspace sizing and dispatch.
// Every check here runs before anything is enqueued; see include/pagedattn.h for the
// contract of each entry point.
#include "pagedattn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa_launch.hpp"
#include "pa_status.hpp"

namespace pa {

thread_local std::string g_last_error;

pa_status_t fail(pa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status_t ok() {
  g_last_error.clear();
  return PA_OK;
}

}  // namespace pa

namespace {

using pa::fail;
using pa::ok;
using pa::g_last_error;

pa_status_t device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PA_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int kv_kind(pa_dtype_t t) {
  switch (t) {
    case PA_F32: return pa::KV_F32;
    case PA_BF16: return pa::KV_BF16;
    case PA_FP8_E5M2: return pa::KV_E5M2;
    case PA_INT8: return pa::KV_I8;
    case PA_FP8_E4M3: return pa::KV_E4M3;
  }
  return -1;
}

bool valid_dtype(int t) {
  return t == PA_F32 || t == PA_BF16 || t == PA_FP8_E5M2 || t == PA_INT8 || t == PA_FP8_E4M3;
}

// Pools with one float32 scale per (token, KV head) after each tile's codes.
bool scaled_dtype(int t) { return t == PA_INT8 || t == PA_FP8_E4M3; }

constexpr int64_t kMaxGridYZ = 65535;

#ifndef PA_LONGEST_FIRST
#define PA_LONGEST_FIRST 1  // dispatch the decode work-groups of long contexts first
#endif
constexpr size_t kWsAlign = 256;

#ifndef PA_PACKED_ONE_LAUNCH
#define PA_PACKED_ONE_LAUNCH 1  // a packed step with prefill chunks and decode tokens: one two-role launch
#endif

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Partition count of the longest context, or 1 when unsplit.
int64_t parts_for(int32_t max_context_len, int32_t partition) {
  if (partition <= 0 || max_context_len <= partition) return 1;
  return (static_cast<int64_t>(max_context_len) + partition - 1) / partition;
}

struct WsLayout {
  size_t o_bytes, ml_bytes, total;
};

// o [rows][hq][parts][D] f32 | m [rows][hq][parts] f32 | l [rows][hq][parts] f32,
// each region 256-byte aligned.
WsLayout ws_layout(int64_t rows, int64_t hkv, int64_t gqa, int64_t head_dim, int64_t parts) {
  WsLayout w{0, 0, 0};
  if (parts <= 1 || rows <= 0) return w;
  const int64_t hq = hkv * gqa;
  w.o_bytes = round_up(static_cast<size_t>(rows * hq * parts * head_dim) * sizeof(float), kWsAlign);
  w.ml_bytes = round_up(static_cast<size_t>(rows * hq * parts) * sizeof(float), kWsAlign);
  w.total = w.o_bytes + 2 * w.ml_bytes;
  return w;
}

int32_t auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  // With at least one (KV head, sequence) context per CU of the current device every context is
  // streamed whole, longest first: no partial results, no merge.  Fewer, longer contexts are
  // split into multiples of 256 tokens, aiming at ~8 work-groups per CU.  Without a device to
  // ask (a host-only process), the MI355X's 256 CUs are assumed.
  const int cus_queried = pa::current_device_cus();
  const int64_t cus = cus_queried > 0 ? cus_queried : 256;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads;
  if (units <= 0 || units >= cus || max_context_len <= 256) return 0;
  int64_t p = static_cast<int64_t>(max_context_len) * units / (8 * cus);
  p = (p + 255) / 256 * 256;
  if (p < 256) p = 256;
  if (p >= max_context_len) return 0;
  return static_cast<int32_t>(p);
}

// Shared checks of the attention calls.  Returns PA_OK and fills `part` / `parts`.
pa_status_t check_attention(const char* fn, int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                            pa_dtype_t q_dtype, pa_dtype_t kv_dtype, int32_t partition_size) {
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_seqs %d < 0", fn, num_seqs);
  if (num_seqs > kMaxGridYZ) return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs %d > 65535", fn, num_seqs);
  if (num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_kv_heads %d <= 0", fn, num_kv_heads);
  if (num_kv_heads > kMaxGridYZ) return fail(PA_ERR_UNSUPPORTED, "%s: num_kv_heads %d > 65535", fn, num_kv_heads);
  if (gqa_group <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: gqa_group %d <= 0", fn, gqa_group);
  if (gqa_group != 1 && gqa_group != 2 && gqa_group != 4 && gqa_group != 8 && gqa_group != 16)
    return fail(PA_ERR_UNSUPPORTED, "%s: gqa_group %d not in {1,2,4,8,16}", fn, gqa_group);
  if (head_dim <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: head_dim %d <= 0", fn, head_dim);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64,128}", fn, head_dim);
  if (block_size <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: block_size %d <= 0", fn, block_size);
  if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d != 16", fn, block_size);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_blocks %d <= 0", fn, num_blocks);
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t(1) << 31))
    return fail(PA_ERR_UNSUPPORTED, "%s: num_blocks * block_size >= 2^31", fn);
  if (max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: max_blocks_per_seq %d <= 0", fn, max_blocks_per_seq);
  if (max_context_len < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: max_context_len %d < 0", fn, max_context_len);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  if (!valid_dtype(q_dtype) || !valid_dtype(kv_dtype))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: unknown dtype (q %d, kv %d)", fn, (int)q_dtype, (int)kv_dtype);
  const bool pair_ok = (q_dtype == PA_F32 && kv_dtype == PA_F32) || (q_dtype == PA_BF16 && kv_dtype == PA_BF16) ||
                       (q_dtype == PA_BF16 && kv_dtype == PA_FP8_E5M2) ||
                       (q_dtype == PA_BF16 && scaled_dtype(kv_dtype));
  if (!pair_ok)
    return fail(PA_ERR_UNSUPPORTED, "%s: (q, kv) dtype pair (%d, %d) not supported", fn, (int)q_dtype,
                (int)kv_dtype);
  if (partition_size < -1)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: partition_size %d < -1", fn, partition_size);
  if (partition_size > 0 && partition_size % block_size != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: partition_size %d is not a multiple of block_size %d", fn,
                partition_size, block_size);
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(pa_status_t s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_ERR_DEVICE: return "device error";
    case PA_ERR_OUT_OF_BLOCKS: return "out of blocks";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

pa_status_t paged_kv_slot_mapping(int32_t* slot_mapping, const int32_t* cu_tokens, const int32_t* end_pos,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                                  int32_t num_tokens, int32_t block_size, int32_t num_blocks,
                                  hipStream_t stream) {
  const char* fn = "paged_kv_slot_mapping";
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_tokens %d < 0", fn, num_tokens);
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_seqs %d < 0", fn, num_seqs);
  if (block_size <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: block_size %d <= 0", fn, block_size);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_blocks %d <= 0", fn, num_blocks);
  if (max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: max_blocks_per_seq %d <= 0", fn, max_blocks_per_seq);
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t(1) << 31))
    return fail(PA_ERR_UNSUPPORTED, "%s: num_blocks * block_size >= 2^31", fn);
  if (num_tokens == 0) return ok();
  if (slot_mapping == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: slot_mapping is null", fn);
  if (num_seqs == 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: %d tokens but no sequences", fn, num_tokens);
  if (cu_tokens == nullptr || end_pos == nullptr || block_tables == nullptr)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: null input pointer", fn);
  if (!aligned(slot_mapping, 4) || !aligned(cu_tokens, 4) || !aligned(end_pos, 4) || !aligned(block_tables, 4))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: int32 arrays must be 4-byte aligned", fn);
  return device_status(pa::launch_slot_mapping(slot_mapping, cu_tokens, end_pos, block_tables, max_blocks_per_seq,
                                               num_seqs, num_tokens, block_size, num_blocks, stream),
                       fn);
}

pa_status_t kv_cache_write(const void* key, const void* value, void* key_cache, void* value_cache,
                           const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, pa_dtype_t src_dtype, pa_dtype_t cache_dtype,
                           hipStream_t stream) {
  const char* fn = "kv_cache_write";
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_tokens %d < 0", fn, num_tokens);
  if (num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_kv_heads %d <= 0", fn, num_kv_heads);
  if (head_dim <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: head_dim %d <= 0", fn, head_dim);
  if (block_size <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: block_size %d <= 0", fn, block_size);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_blocks %d <= 0", fn, num_blocks);
  if (!valid_dtype(src_dtype) || !valid_dtype(cache_dtype))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: unknown dtype (src %d, cache %d)", fn, (int)src_dtype,
                (int)cache_dtype);
  const bool pair_ok = (src_dtype == PA_F32 && cache_dtype == PA_F32) ||
                       (src_dtype == PA_BF16 && cache_dtype == PA_BF16) ||
                       (src_dtype == PA_BF16 && cache_dtype == PA_FP8_E5M2) ||
                       (src_dtype == PA_BF16 && scaled_dtype(cache_dtype));
  if (!pair_ok)
    return fail(PA_ERR_UNSUPPORTED, "%s: (src, cache) dtype pair (%d, %d) not supported", fn, (int)src_dtype,
                (int)cache_dtype);
  if (scaled_dtype(cache_dtype) && (block_size != 16 || (head_dim != 64 && head_dim != 128)))
    return fail(PA_ERR_UNSUPPORTED, "%s: an INT8 / FP8_E4M3 pool takes block_size 16 and head_dim 64 or 128", fn);
  const int src_sz = src_dtype == PA_F32 ? 4 : 2;
  if ((static_cast<int64_t>(head_dim) * src_sz) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d rows are not a multiple of 16 bytes", fn, head_dim);
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t(1) << 31))
    return fail(PA_ERR_UNSUPPORTED, "%s: num_blocks * block_size >= 2^31", fn);
  if (static_cast<int64_t>(num_tokens) * num_kv_heads * head_dim * src_sz / 16 >= (int64_t(1) << 40))
    return fail(PA_ERR_UNSUPPORTED, "%s: write too large", fn);
  if (num_tokens == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
  if (!aligned(key, 16) || !aligned(value, 16))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: key/value must be 16-byte aligned", fn);
  const size_t cache_align = cache_dtype == PA_FP8_E5M2 ? 8 : 16;  // INT8 tiles: 16-byte steps
  if (!aligned(key_cache, cache_align) || !aligned(value_cache, cache_align))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: caches must be %zu-byte aligned", fn, cache_align);
  if (!aligned(slot_mapping, 4)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: slot_mapping misaligned", fn);
  return device_status(pa::launch_cache_write(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                              num_kv_heads, head_dim, block_size, num_blocks, kv_kind(src_dtype),
                                              kv_kind(cache_dtype), stream),
                       fn);
}

int32_t paged_attention_auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                       int32_t max_context_len) {
  (void)gqa_group;
  (void)head_dim;
  return auto_partition(num_seqs, num_kv_heads, max_context_len);
}

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                      int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || gqa_group <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int32_t part = partition_size == -1 ? auto_partition(num_seqs, num_kv_heads, max_context_len)
                                            : partition_size;
  const int64_t parts = parts_for(max_context_len, part);
  return ws_layout(num_seqs, num_kv_heads, gqa_group, head_dim, parts).total;
}

}  // extern "C"

namespace {

// Checks shared by the decode calls that read the cache, and the launch parameters.
pa_status_t prepare_decode(const char* fn, pa::DecodeParams& p, void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                           float scale, pa_dtype_t q_dtype, pa_dtype_t kv_dtype, int32_t partition_size,
                           void* workspace, size_t workspace_bytes, bool needs_cache) {
  pa_status_t st = check_attention(fn, num_seqs, num_kv_heads, gqa_group, head_dim, block_size, num_blocks,
                                   max_blocks_per_seq, max_context_len, scale, q_dtype, kv_dtype, partition_size);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  if (!out || !context_lens) return fail(PA_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
  if (needs_cache && (!query || !key_cache || !value_cache || !block_tables))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
  if (!aligned(out, 16) || (needs_cache && !aligned(query, 16)))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: query/out must be 16-byte aligned", fn);
  if (needs_cache && (!aligned(key_cache, 16) || !aligned(value_cache, 16)))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: caches must be 16-byte aligned", fn);
  if ((needs_cache && !aligned(block_tables, 4)) || !aligned(context_lens, 4))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: int32 arrays must be 4-byte aligned", fn);
  const int32_t part = partition_size == -1 ? auto_partition(num_seqs, num_kv_heads, max_context_len)
                                            : partition_size;
  const int64_t parts = parts_for(max_context_len, part);
  const WsLayout ws = ws_layout(num_seqs, num_kv_heads, gqa_group, head_dim, parts);
  if (ws.total > 0) {
    if (workspace == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: workspace is null, need %zu bytes", fn, ws.total);
    if (workspace_bytes < ws.total)
      return fail(PA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, ws.total);
    if (!aligned(workspace, kWsAlign)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", fn);
  }
  if (parts > kMaxGridYZ) return fail(PA_ERR_UNSUPPORTED, "%s: %lld partitions > 65535", fn, (long long)parts);
  p = pa::DecodeParams{};
  p.out = out;
  p.ws_o = ws.total ? static_cast<float*>(workspace) : nullptr;
  p.ws_m = ws.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.o_bytes) : nullptr;
  p.ws_l = ws.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.o_bytes + ws.ml_bytes) : nullptr;
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.cu_q = nullptr;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.num_kv_heads = num_kv_heads;
  p.max_context_len = max_context_len;
  p.partition_tokens = parts > 1 ? part : 0;
  p.max_parts = static_cast<int32_t>(parts);
  p.scale_log2 = scale * 1.4426950408889634f;
  // longest-first only pays when whole contexts are the work units (see decode.hip)
  p.longest_first = PA_LONGEST_FIRST && parts <= 1 && num_seqs <= pa::kLongestFirstMaxSeqs;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t paged_attention_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                                   int32_t gqa_group, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_context_len, float scale, pa_dtype_t q_dtype, pa_dtype_t kv_dtype,
                                   int32_t partition_size, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  const char* fn = "paged_attention_decode";
  pa::DecodeParams p;
  pa_status_t st = prepare_decode(fn, p, out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                                  context_lens, num_seqs, num_kv_heads, gqa_group, head_dim, block_size, num_blocks,
                                  max_context_len, scale, q_dtype, kv_dtype, partition_size, workspace,
                                  workspace_bytes, true);
  if (st != PA_OK || num_seqs == 0) return st == PA_OK ? ok() : st;
  hipError_t e = pa::launch_decode_partitions(p, kv_kind(kv_dtype), head_dim, gqa_group, num_seqs, stream);
  if (e == hipSuccess) e = pa::launch_decode_reduce(p, q_dtype == PA_BF16, head_dim, num_kv_heads * gqa_group,
                                                    num_seqs, stream);
  return device_status(e, fn);
}

static_assert(pa::kStaticWorkspaceBytes == PA_STATIC_WORKSPACE_BYTES, "scratch size of the header and the library");

pa_status_t paged_attention_decode_static(void* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                          int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                                          float scale, pa_dtype_t q_dtype, pa_dtype_t kv_dtype,
                                          int32_t partition_size, hipStream_t stream) {
  const char* fn = "paged_attention_decode_static";
  pa_status_t st = check_attention(fn, num_seqs, num_kv_heads, gqa_group, head_dim, block_size, num_blocks,
                                   max_blocks_per_seq, max_context_len, scale, q_dtype, kv_dtype, partition_size);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  const size_t need = paged_attention_workspace_size(num_seqs, num_kv_heads, gqa_group, head_dim, max_context_len,
                                                     partition_size);
  if (need > PA_STATIC_WORKSPACE_BYTES)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "%s: the split needs %zu bytes of scratch, the library holds %zu", fn,
                need, static_cast<size_t>(PA_STATIC_WORKSPACE_BYTES));
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = pa::static_workspace(&ws);
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "%s: scratch address: %s", fn, hipGetErrorString(e));
  }
  pa::DecodeParams p;
  st = prepare_decode(fn, p, out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                      num_seqs, num_kv_heads, gqa_group, head_dim, block_size, num_blocks, max_context_len, scale,
                      q_dtype, kv_dtype, partition_size, ws, need > 0 ? PA_STATIC_WORKSPACE_BYTES : 0, true);
  if (st != PA_OK) return st;
  hipError_t e = pa::launch_decode_partitions(p, kv_kind(kv_dtype), head_dim, gqa_group, num_seqs, stream);
  if (e == hipSuccess) e = pa::launch_decode_reduce(p, q_dtype == PA_BF16, head_dim, num_kv_heads * gqa_group,
                                                    num_seqs, stream);
  return device_status(e, fn);
}

pa_status_t paged_attention_decode_partitions(void* out, const void* query, const void* key_cache,
                                              const void* value_cache, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                                              int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                              int32_t max_context_len, float scale, pa_dtype_t q_dtype,
                                              pa_dtype_t kv_dtype, int32_t partition_size, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "paged_attention_decode_partitions";
  pa::DecodeParams p;
  pa_status_t st = prepare_decode(fn, p, out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                                  context_lens, num_seqs, num_kv_heads, gqa_group, head_dim, block_size, num_blocks,
                                  max_context_len, scale, q_dtype, kv_dtype, partition_size, workspace,
                                  workspace_bytes, true);
  if (st != PA_OK || num_seqs == 0) return st == PA_OK ? ok() : st;
  return device_status(pa::launch_decode_partitions(p, kv_kind(kv_dtype), head_dim, gqa_group, num_seqs, stream), fn);
}

pa_status_t paged_attention_decode_reduce(void* out, const int32_t* context_lens, int32_t max_blocks_per_seq,
                                          int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                                          int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                          pa_dtype_t q_dtype, pa_dtype_t kv_dtype, int32_t partition_size,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "paged_attention_decode_reduce";
  pa::DecodeParams p;
  pa_status_t st = prepare_decode(fn, p, out, nullptr, nullptr, nullptr, nullptr, max_blocks_per_seq, context_lens,
                                  num_seqs, num_kv_heads, gqa_group, head_dim, block_size, 1, max_context_len, 1.0f,
                                  q_dtype, kv_dtype, partition_size, workspace, workspace_bytes, false);
  if (st != PA_OK || num_seqs == 0) return st == PA_OK ? ok() : st;
  return device_status(pa::launch_decode_reduce(p, q_dtype == PA_BF16, head_dim, num_kv_heads * gqa_group, num_seqs,
                                                stream),
                       fn);
}

pa_status_t paged_attention_decode_append(void* out, const void* query, const void* key, const void* value,
                                          void* key_cache, void* value_cache, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                          int32_t block_size, int32_t num_blocks, int32_t max_context_len, float scale,
                                          pa_dtype_t q_dtype, pa_dtype_t kv_dtype, int32_t partition_size,
                                          int32_t flags, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  const char* fn = "paged_attention_decode_append";
  if (flags & ~PA_APPEND_SKIP_REDUCE) return fail(PA_ERR_INVALID_ARGUMENT, "%s: unknown flags 0x%x", fn, flags);
  pa::DecodeParams p;
  pa_status_t st = prepare_decode(fn, p, out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                                  context_lens, num_seqs, num_kv_heads, gqa_group, head_dim, block_size, num_blocks,
                                  max_context_len, scale, q_dtype, kv_dtype, partition_size, workspace,
                                  workspace_bytes, true);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  if (!key || !value) return fail(PA_ERR_INVALID_ARGUMENT, "%s: null key/value row pointer", fn);
  if (!aligned(key, 16) || !aligned(value, 16))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: key/value rows must be 16-byte aligned", fn);
  p.key_new = key;
  p.value_new = value;
  p.key_cache_w = key_cache;
  p.value_cache_w = value_cache;
  hipError_t e = pa::launch_decode_partitions(p, kv_kind(kv_dtype), head_dim, gqa_group, num_seqs, stream);
  if (e == hipSuccess && !(flags & PA_APPEND_SKIP_REDUCE))
    e = pa::launch_decode_reduce(p, q_dtype == PA_BF16, head_dim, num_kv_heads * gqa_group, num_seqs, stream);
  return device_status(e, fn);
}

pa_status_t paged_attention_varlen(void* out, const void* query, const void* key_cache, const void* value_cache,
                                   const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                                   int32_t total_q, int32_t max_q_len, int32_t num_kv_heads, int32_t gqa_group,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                                   float scale, int32_t causal, pa_dtype_t q_dtype, pa_dtype_t kv_dtype,
                                   int32_t partition_size, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  const char* fn = "paged_attention_varlen";
  if (total_q < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: total_q %d < 0", fn, total_q);
  if (max_q_len < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: max_q_len %d < 0", fn, max_q_len);
  if (max_q_len > total_q) return fail(PA_ERR_INVALID_ARGUMENT, "%s: max_q_len %d > total_q %d", fn, max_q_len, total_q);
  if (causal != 0 && causal != 1) return fail(PA_ERR_INVALID_ARGUMENT, "%s: causal must be 0 or 1", fn);
  pa::DecodeParams p;
  pa_status_t st = prepare_decode(fn, p, out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                                  context_lens, num_seqs, num_kv_heads, gqa_group, head_dim, block_size, num_blocks,
                                  max_context_len, scale, q_dtype, kv_dtype, partition_size, workspace,
                                  workspace_bytes, true);
  if (st != PA_OK) return st;
  if (q_dtype != PA_BF16 || (kv_dtype != PA_BF16 && kv_dtype != PA_FP8_E5M2))
    return fail(PA_ERR_UNSUPPORTED, "%s: packed batches take bf16 queries and a bf16 or FP8_E5M2 cache", fn);
  if (num_seqs == 0 || total_q == 0) return ok();
  if (!cu_seqlens_q || !aligned(cu_seqlens_q, 4)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens_q", fn);
  const int64_t prefill_tiles = (static_cast<int64_t>(max_q_len) * gqa_group + 127) / 128;
  if (prefill_tiles > kMaxGridYZ) return fail(PA_ERR_UNSUPPORTED, "%s: max_q_len %d too large", fn, max_q_len);
  p.cu_q = cu_seqlens_q;
  p.causal = causal;
  // Every sequence holds at most max_q_len of the total_q rows, so when total_q equals
  // num_seqs * max_q_len >= 2 * num_seqs none has a single row: no decode launch.
  const bool single_rows = !(max_q_len >= 2 && static_cast<int64_t>(total_q) == static_cast<int64_t>(num_seqs) * max_q_len);
  hipError_t e = hipSuccess;
  const bool prefill_rows = max_q_len >= 2 && !pa::multiquery_applies(gqa_group, max_q_len);
  if (PA_PACKED_ONE_LAUNCH && single_rows && prefill_rows && pa::packed_step_applies(p, num_seqs, max_q_len)) {
    // decode tokens and prefill chunks together: one two-role launch
    return device_status(pa::launch_packed_step(p, kv_kind(kv_dtype), head_dim, gqa_group, num_seqs, total_q,
                                                max_q_len, stream),
                         fn);
  }
  if (single_rows) {
    e = pa::launch_decode_partitions(p, kv_kind(kv_dtype), head_dim, gqa_group, num_seqs, stream);
    if (e == hipSuccess) e = pa::launch_decode_reduce(p, true, head_dim, num_kv_heads * gqa_group, num_seqs, stream);
  }
  if (e == hipSuccess && max_q_len >= 2) {  // some sequence may have several rows
    if (pa::multiquery_applies(gqa_group, max_q_len))
      e = pa::launch_varlen_multiquery(p, kv_kind(kv_dtype), head_dim, gqa_group, num_seqs, max_q_len, stream);
    else
      e = pa::launch_varlen_prefill(p, kv_kind(kv_dtype), head_dim, gqa_group, num_seqs, total_q, max_q_len, stream);
  }
  return device_status(e, fn);
}

pa_status_t paged_kv_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int32_t num_pairs,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 pa_dtype_t cache_dtype, hipStream_t stream) {
  const char* fn = "paged_kv_copy_blocks";
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_pairs %d < 0", fn, num_pairs);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_kv_heads, head_dim, block_size and num_blocks must be > 0", fn);
  if (!valid_dtype(cache_dtype)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: unknown cache dtype %d", fn, (int)cache_dtype);
  if (scaled_dtype(cache_dtype) && block_size != 16)
    return fail(PA_ERR_UNSUPPORTED, "%s: an INT8 / FP8_E4M3 pool takes block_size 16", fn);
  const size_t elem = cache_dtype == PA_F32 ? 4 : cache_dtype == PA_BF16 ? 2 : 1;
  // a scaled key tile carries a key and a value float32 scale per token after its codes
  const size_t v_block_bytes = static_cast<size_t>(num_kv_heads) * block_size * head_dim * elem;
  const size_t k_block_bytes =
      v_block_bytes + (scaled_dtype(cache_dtype) ? static_cast<size_t>(num_kv_heads) * block_size * 8 : 0);
  if (k_block_bytes % 16 != 0 || v_block_bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: a block of %zu bytes is not a multiple of 16", fn, v_block_bytes);
  if (num_pairs == 0) return ok();
  if (!key_cache || !value_cache || !pairs) return fail(PA_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(pairs, 4))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: caches must be 16-byte aligned", fn);
  return device_status(
      pa::launch_copy_blocks(key_cache, value_cache, pairs, num_pairs, k_block_bytes, v_block_bytes, num_blocks, stream),
      fn);
}

}  // extern "C"
