// Internal launch interface between the host C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Element type of a pool (values match pa_dtype_t).
// KV_I8, KV_E4M3: 8-bit codes with one float32 scale per (token, KV head) after each (block,
// head) tile ("scaled" kinds)
enum KvKind : int { KV_F32 = 0, KV_BF16 = 1, KV_E5M2 = 2, KV_I8 = 3, KV_E4M3 = 4 };

struct DecodeParams {
  void* out;
  float* ws_o;  // [rows][hq][max_parts][D]
  float* ws_m;  // [rows][hq][max_parts]
  float* ws_l;  // [rows][hq][max_parts]
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q;  // null: decode batch (query row s); else packed varlen rows
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t max_context_len;
  int32_t partition_tokens;  // 0: one pass per context
  int32_t max_parts;         // grid.x: partitions of the longest context (1 if unsplit)
  float scale_log2;          // scale * log2(e)
  // Append mode (non-null key_new): each sequence's newest token (position L-1) has its
  // K/V row [num_kv_heads][D] (query dtype) in key_new/value_new; the work-group whose
  // partition holds that position writes it into the pools and uses it directly.
  const void* key_new;
  const void* value_new;
  void* key_cache_w;
  void* value_cache_w;
  // Longest-first order: grid z is a rank, not a sequence index; every work-group ranks
  // the sequences by context length (ties by index) and takes the one with its rank, so
  // the dispatcher hands out long contexts first (greedy longest-processing-time).
  int32_t longest_first;
  // With longest_first, when every work-group of the grid is resident at once (the launcher
  // checks the occupancy): the number of CUs.  Work-groups i and i + snake share a CU, so
  // rank order is reversed on every second lap of this length, pairing long contexts with
  // short ones on each CU.  0: plain rank order.
  int32_t snake;
  // Decode kernel: work-groups resident at once (from the occupancy); the snake order is applied
  // when the units of the sequences that take part fit in it (the kernel counts them).
  int32_t resident;
  int32_t causal;  // packed (varlen) batches: mask aligned to the end of each context
  // Prefill kernel: number of sequences to rank into the longest-first unit order (the grid
  // is then one-dimensional); 0: natural three-dimensional order.
  int32_t sched_seqs;
};

// Partition pass: a sequence with one partition gets its output row; a split one gets
// (o/l, m, l) per partition in the workspace.
hipError_t launch_decode_partitions(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs,
                                    hipStream_t stream);
// Compute units of the current device (0 when it cannot be queried).
int current_device_cus();

// Bytes of the split-KV scratch array the library holds on every GPU (the decode entry point
// that allocates nothing); equals PA_STATIC_WORKSPACE_BYTES of the public header.
constexpr size_t kStaticWorkspaceBytes = size_t(32) << 20;
// Device address of that array on the current device (looked up once per device).
hipError_t static_workspace(void** ptr);

// Merge pass over the split sequences (no-op when p.max_parts <= 1).
hipError_t launch_decode_reduce(const DecodeParams& p, bool out_bf16, int head_dim, int num_q_heads, int num_seqs,
                                hipStream_t stream);

// Longest-first order (every work-group ranks the batch's sequences by length) is used up to this
// many sequences, and by the decode and multi-query launchers only when every unit of the grid is
// resident at once, where the snake order pairs long and short contexts on each CU.  The ranking
// costs each work-group O(n^2 / threads); measured on bf16 decode batches (4 query heads per KV
// head) against the plain grid order: 61.1 against 64.9 us at 64 sequences (resident), but 65.8
// against 63.5 at 128, 140 against 116 at 256, and 2131 against 146 us at 1024.
constexpr int kLongestFirstMaxSeqs = 128;

// The decode calls (no packed rows) over a bf16 or E5M2 cache with 8 or 16 query heads per KV head:
// the partition pass on MFMA (multiquery.hip), same grid, workspace and append as the vector one.
bool decode_mfma_applies(const DecodeParams& p, int kv_kind, int head_dim, int gqa);
hipError_t launch_decode_mfma(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs,
                              hipStream_t stream);

// Multi-token rows of a packed batch when every sequence has at most max_q_len tokens and
// max_q_len * gqa <= 32 (speculative verification): one work-group streams each context once.
bool multiquery_applies(int gqa, int max_q_len);
hipError_t launch_varlen_multiquery(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs,
                                    int max_q_len, hipStream_t stream);

// Prefill rows (sequences with >= 2 query tokens) of a packed batch, on MFMA (bf16 or E5M2 cache).
hipError_t launch_varlen_prefill(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs, int total_q,
                                 int max_q_len, hipStream_t stream);

// A packed step with both prefill chunks and decode tokens as one two-role launch (whole-context
// decode passes only, at most 1024 sequences).
bool packed_step_applies(const DecodeParams& p, int num_seqs, int max_q_len);
hipError_t launch_packed_step(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs, int total_q,
                              int max_q_len, hipStream_t stream);

hipError_t launch_slot_mapping(int32_t* slots, const int32_t* cu, const int32_t* end_pos,
                               const int32_t* tables, int32_t max_blocks, int32_t num_seqs,
                               int32_t num_tokens, int32_t block_size, int32_t num_blocks,
                               hipStream_t stream);

// Copy whole blocks src -> dst of both pools (pairs: device int32 [2 * num_pairs]); a key block
// and a value block may differ in size (the scaled kinds keep both rows' scales in the key pool).
hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int32_t num_pairs,
                              size_t k_block_bytes, size_t v_block_bytes, int32_t num_blocks, hipStream_t stream);

hipError_t launch_cache_write(const void* key, const void* value, void* key_cache, void* value_cache,
                              const int32_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks, int src_kind,
                              int cache_kind, hipStream_t stream);

}  // namespace pa
