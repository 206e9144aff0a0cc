/*
 * libpagedattn -- PagedAttention over a blocked KV cache, for AMD MI355X (gfx950).
 *
 * The operations follow these pages (cited by title and section):
 *   [CI]  Colossal-Inference release post ("AI大模型推理速度翻倍，Colossal-Inference开源发布"),
 *         sections "分块式KV缓存 (BlockedKeyValueCache)", "KV缓存量化 (KVCache Quant)",
 *         "分页注意力算法 (PagedAttention)", "连续批量化算法 (Continuous Batching)".
 *   [OPT] LLM inference optimisation overview ("AI 大模型推理优化技术详解"),
 *         sections 2.1.2 "Paged Attention", 2.2.1 "Flash Attention", 2.2.2 "GQA",
 *         2.4 "服务" (Continuous Batching, Dynamic Batching).
 *   [TACO] Taco-LLM article ("易用性对齐 vLLM，推理效率提升超200%，这款国产加速框架什么来头？"),
 *         section "使用 Prefix Cache 技术降低 TTFT".
 *   [FW]  LLM inference frameworks overview (vLLM, LMDeploy, ...), section "LMDeploy": KV cache
 *         INT8 quantisation; [OPT] 2.6 "低比特量化": low-bit formats cut memory and traffic.
 *
 * Data model
 *   Every sequence's keys and values live in fixed-size blocks of `block_size`
 *   tokens taken from a shared pool; a per-sequence block table maps logical
 *   block j (tokens j*B .. j*B+B-1) to a physical block id [CI BlockedKeyValueCache,
 *   OPT 2.1.2].  Several tables may name the same physical block (a shared prefix).
 *
 *   Pool layout (key and value pools alike), row-major:
 *       cache[num_blocks][num_kv_heads][block_size][head_dim]
 *   so one (block, kv head) tile of block_size x head_dim elements is contiguous.
 *
 *   Query head h reads KV head h / gqa_group  [OPT 2.2.2; the grouping is taken
 *   as contiguous].  num_q_heads = num_kv_heads * gqa_group.
 *   Queries and outputs are row-major [rows][num_q_heads][head_dim].
 *
 * Element types
 *   PA_F32   IEEE binary32
 *   PA_BF16  bfloat16 (upper half of a binary32); outputs are rounded to nearest even
 *   PA_FP8_E5M2  1 sign, 5 exponent (bias 15), 2 mantissa bits, with inf and NaN; the
 *            cache write casts bf16 -> E5M2 by round-to-nearest-even without saturation
 *            (|x| >= 61440 -> inf, NaN -> sign|0x7F); reads widen exactly
 *            [CI KVCache Quant: cast on store, cast back on load].
 *   PA_INT8  symmetric int8 codes with one float32 scale per (token, KV head) row
 *            [FW LMDeploy: KV cache INT8; no page fixes the scheme, this is the library's].
 *            The cache write computes, in float32 with round-to-nearest-even:
 *                amax = max_d |x_d| (NaN elements ignored), inv = amax > 0 ? 127 / amax : 0,
 *                code_d = clamp(rint(x_d * inv), -127, 127) (a NaN product gives -127),
 *                scale = amax / 127;
 *            a reader uses code * scale.  Pool layout (block_size must be 16), key and value
 *            pools differing:
 *                key_cache[num_blocks][num_kv_heads][16 * head_dim + 128] bytes
 *                value_cache[num_blocks][num_kv_heads][16][head_dim] bytes
 *            each (block, KV head) key tile holding the 16 x head_dim key codes (token-major, as
 *            in the other pools), then the 16 float32 key scales, then the 16 float32 value
 *            scales of the same tokens; the value tile holds the value codes only.  Within each
 *            group of 16 scales the scale of token t sits at float index 4 * (t % 4) + t / 4 (so
 *            the scales of tokens r, r+4, r+8, r+12 are one 16-byte word).  Every tile is a
 *            whole number of 128-byte lines, and both rows' scales travel with the key tile a
 *            work-group reads anyway.  Decode reads the codes as f16 and forms, per token, the
 *            probability times the value scale in f16 (11 significant bits; p <= 256 with
 *            the kernel's lazy running max): value rows need amax below 32000, and
 *            products below 2^-14 keep only f16's subnormal precision.
 *   PA_FP8_E4M3  scaled FP8: OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
 *            bits, no infinities, largest finite 448, S.1111.111 = NaN) of each (token, KV head)
 *            row scaled to the format's range, with one float32 scale per row [OPT 2.6; the
 *            scheme is this library's].  The cache write computes, in float32: amax as for
 *            INT8, inv = amax > 0 ? 448 / amax : 0, code_d = x_d * inv rounded to the nearest
 *            E4M3 value (ties to the even code, saturating at 448; a NaN product gives 0x7F),
 *            scale = amax / 448; a reader uses value(code) * scale.  Pool layout as for INT8.
 *            Decode widens codes to f16 exactly and applies the scales as for INT8 (value rows
 *            need amax below 114000 for the f16 weights).
 *
 * Conventions for every entry point
 *   - All pointers are device pointers unless stated; the caller owns every buffer.
 *     The library never allocates or frees device memory and never synchronises.  Its
 *     state is a thread-local error string, the host objects a caller creates and
 *     destroys (block managers, schedulers) and one fixed scratch array per GPU that only
 *     paged_attention_decode_static uses; the other attention and cache calls are re-entrant.
 *   - Work is enqueued on `stream`; calls return before the device has finished.
 *   - Scalar arguments and pointer alignment are checked on the host before anything
 *     is enqueued: a bad value returns PA_ERR_INVALID_ARGUMENT, a well-formed but
 *     unsupported combination PA_ERR_UNSUPPORTED, and nothing is launched.  A launch
 *     failure returns PA_ERR_DEVICE.  pa_last_error() gives the reason in words.
 *   - Device contents (table entries, lengths, slots) are not validated on the host.
 *     Kernels stay in bounds regardless: a table entry outside [0, num_blocks), a
 *     slot outside the pool or a position past the table is skipped (its token
 *     contributes nothing / its row is not written); context lengths are clamped to
 *     [0, min(max_context_len, max_blocks_per_seq * block_size)].  Results for such
 *     inputs are unspecified but no access leaves the buffers described here.
 *   - Supported now: block_size 16; head_dim 64 or 128; gqa_group 1, 2, 4, 8 or 16;
 *     (query, cache) types (F32, F32), (BF16, BF16), (BF16, FP8_E5M2), (BF16, FP8_E4M3) and
 *     (BF16, INT8) for the decode calls; packed (varlen) batches take (BF16, BF16) and
 *     (BF16, FP8_E5M2).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 5

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,
  PA_ERR_UNSUPPORTED = 2,
  PA_ERR_WORKSPACE_TOO_SMALL = 3,
  PA_ERR_DEVICE = 4,
  PA_ERR_OUT_OF_BLOCKS = 5
} pa_status_t;

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E5M2 = 2, PA_INT8 = 3, PA_FP8_E4M3 = 4 } pa_dtype_t;

/* Version of this header's ABI (PA_ABI_VERSION). */
int pa_abi_version(void);

/* Static text naming a status code. */
const char* pa_status_string(pa_status_t status);

/* Reason for the last failing call on this host thread ("" after a success).  The
 * string stays valid until the next call on the same thread. */
const char* pa_last_error(void);

/*
 * paged_kv_slot_mapping -- the pool slot of every packed token row.
 * [CI BlockedKeyValueCache: logical blocks reach physical blocks through the block
 *  table; OPT 2.1.2: block size 16 by default]
 *
 * Sequence s owns packed rows cu_tokens[s] .. cu_tokens[s+1]-1 (n_s rows); row i of
 * them is the token at logical position p = end_pos[s] - n_s + i, and
 *     slot_mapping[row] = block_tables[s][p / block_size] * block_size + p % block_size.
 * A row whose position is negative or past the table, or whose table entry is not in
 * [0, num_blocks), gets -1 (a cache write skips it).  Rows not covered by
 * cu_tokens[0] .. cu_tokens[num_seqs] also get -1.
 *
 *   slot_mapping  out, int32 [num_tokens]
 *   cu_tokens     int32 [num_seqs + 1], non-decreasing, cu_tokens[0] = 0
 *   end_pos       int32 [num_seqs]: one past the last written position of each sequence
 *                 (the context length when the rows are a step's newest tokens)
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]
 *   num_blocks * block_size must be below 2^31.
 */
pa_status_t paged_kv_slot_mapping(int32_t* slot_mapping, const int32_t* cu_tokens,
                                  const int32_t* end_pos, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, int32_t num_seqs,
                                  int32_t num_tokens, int32_t block_size, int32_t num_blocks,
                                  hipStream_t stream);

/*
 * kv_cache_write -- scatter new key/value rows into the pools ("kernel 1").
 * [CI BlockedKeyValueCache; CI KVCache Quant: the writer casts to E5M2 on store;
 *  FW LMDeploy: INT8 KV cache]
 *
 *   key, value    [num_tokens][num_kv_heads][head_dim] of src_dtype, dense, 16-byte
 *                 aligned
 *   key_cache,
 *   value_cache   [num_blocks][num_kv_heads][block_size][head_dim] of cache_dtype
 *   slot_mapping  int32 [num_tokens]; row r goes to block slot/block_size, offset
 *                 slot % block_size; slot < 0 or >= num_blocks*block_size skips the row
 *   (src, cache) in {(F32, F32), (BF16, BF16), (BF16, FP8_E5M2), (BF16, INT8), (BF16,
 *   FP8_E4M3)}; a same-type write copies bits, the E5M2 cast is round-to-nearest-even, an INT8
 *   or FP8_E4M3 write quantises each (token, KV head) row and stores its codes and scale (see
 *   above: both scales go to the key pool; block_size 16 and head_dim 64 or 128 for these).
 *   Two rows with the same slot in one call race: the stored row is unspecified.
 */
pa_status_t kv_cache_write(const void* key, const void* value, void* key_cache,
                           void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, pa_dtype_t src_dtype, pa_dtype_t cache_dtype,
                           hipStream_t stream);

/*
 * paged_attention_workspace_size -- bytes of device workspace that
 * paged_attention_decode / paged_attention_varlen need for these arguments
 * (0 when no sequence is split).  `partition_size` as in paged_attention_decode
 * (-1 resolves the same way the attention call will).
 *
 * Workspace layout, with P = partitions of the longest context and R = num_seqs, each
 * region starting on a 256-byte boundary (scratch: nothing carries over between calls):
 *   o  float [R][num_q_heads][P][head_dim]   partition outputs, already divided by l
 *   m  float [R][num_q_heads][P]             partition max of scale*log2(e)*q.k
 *   l  float [R][num_q_heads][P]             partition sum of 2^(score - m)
 */
size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                      int32_t gqa_group, int32_t head_dim,
                                      int32_t max_context_len, int32_t partition_size);

/* The partition size (tokens) that partition_size = -1 resolves to on the current device: 0 (one
 * pass per context) when the (sequence, KV head) contexts are at least the device's CU count,
 * otherwise a multiple of 256 tokens aiming at about 8 work-groups per CU (256 CUs are assumed
 * when no device can be queried). */
int32_t paged_attention_auto_partition(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t gqa_group, int32_t head_dim,
                                       int32_t max_context_len);

/*
 * paged_attention_decode -- single-token decode attention over the blocked cache
 * ("kernel 2").  [CI PagedAttention: decode attention is a memory-bound GEMV over the
 * cached keys and values, read block by block through the table; OPT 2.2.2 GQA;
 * OPT 2.2.1: softmax reduced without the whole input, used for split-KV]
 *
 * For sequence s with L = context_lens[s] (the current token included) and query
 * head h (KV head g = h / gqa_group):
 *   S_t = scale * q[s][h] . K_s[t][g],   t < L
 *   out[s][h] = sum_t exp(S_t - max S) V_s[t][g] / sum_t exp(S_t - max S)
 * where K_s[t] is row t % block_size of physical block block_tables[s][t / block_size].
 * L = 0 gives a zero row.
 *
 *   out           [num_seqs][num_kv_heads*gqa_group][head_dim], q_dtype
 *   query         [num_seqs][num_kv_heads*gqa_group][head_dim], q_dtype, 16-byte aligned
 *   key_cache,
 *   value_cache   pools as above, kv_dtype
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entries past ceil(L/B) unread
 *   context_lens  int32 [num_seqs]
 *   max_context_len  host-side upper bound of context_lens (sizes the launch)
 *   partition_size   0: one pass over each whole context; > 0 (multiple of block_size):
 *                    split every context into partitions of that many tokens, each
 *                    written to the workspace and merged by a second kernel;
 *                    -1: chosen by the library (paged_attention_auto_partition)
 *   workspace     device buffer of at least paged_attention_workspace_size(...) bytes
 *                 (may be NULL when that size is 0), 256-byte aligned; its contents
 *                 are scratch, overwritten on every call
 * Query range over 8-bit caches: with an FP8_E5M2, INT8 or FP8_E4M3 cache the bf16 query is
 * taken to f16 for the dot products.  That is exact for elements of magnitude 2^-14 .. 65280
 * (every bf16 value f16 can hold); smaller elements keep f16's subnormal precision.  Queries must
 * stay below 65536 in magnitude on these caches: a larger element overflows to inf, and the output
 * row of its (sequence, head) is then unspecified (zero or not finite, by path); every other head
 * and sequence is unaffected.
 * Probabilities: with gqa_group 8 or 16 over a BF16 or FP8_E5M2 cache the dot products run on the
 * matrix cores, and the probabilities enter the value product and the row sum rounded to bf16
 * (f16 over FP8_E5M2), the same rounded values in both; the other shapes keep them in fp32 for a
 * bf16 or f32 cache.  The partials m and l above follow the same rule.
 */
pa_status_t paged_attention_decode(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_context_len, float scale, pa_dtype_t q_dtype,
                                   pa_dtype_t kv_dtype, int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_static -- paged_attention_decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks and result as paged_attention_decode, without the workspace:
 * the split-KV partials go to a scratch array the library holds on every GPU it runs on, until the
 * process ends (PA_STATIC_WORKSPACE_BYTES per GPU).  A call whose split needs more scratch than
 * that (paged_attention_workspace_size(...) > PA_STATIC_WORKSPACE_BYTES) returns
 * PA_ERR_WORKSPACE_TOO_SMALL and launches nothing.  The call allocates and frees nothing.
 * Every call on one GPU uses that GPU's one array, which keeps the last call's partials (nothing in
 * it has to start at zero: a call writes every partial it reads): two calls that overlap on one GPU
 * (on different streams, or from different host threads without ordering) race on it, and the
 * caller orders them (one stream, or events).
 */
#define PA_STATIC_WORKSPACE_BYTES (32u << 20)

pa_status_t paged_attention_decode_static(void* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                          int32_t max_context_len, float scale, pa_dtype_t q_dtype,
                                          pa_dtype_t kv_dtype, int32_t partition_size, hipStream_t stream);

/*
 * The two passes of paged_attention_decode, for callers that schedule or time them
 * apart.  Called one after the other on one stream with the same arguments they are
 * exactly paged_attention_decode.
 *
 * paged_attention_decode_partitions -- the streaming pass.  Every sequence with at most
 *   one partition gets its output row; every split sequence gets, per query head and
 *   partition, the partition's normalised output, max and sum in the workspace (layout
 *   above).  [CI PagedAttention; OPT 2.2.1]
 * paged_attention_decode_reduce -- the merge pass of split-KV: for each split sequence
 *   and query head, M = max_j m_j, w_j = 2^(m_j - M) l_j, out = sum_j w_j o_j / sum_j w_j
 *   (the running max / sum identity of OPT 2.2.1).  Does nothing when no sequence is
 *   split.  Arguments mean what they mean in paged_attention_decode.
 */
pa_status_t paged_attention_decode_partitions(void* out, const void* query, const void* key_cache,
                                              const void* value_cache, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                                              int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                              int32_t max_context_len, float scale, pa_dtype_t q_dtype,
                                              pa_dtype_t kv_dtype, int32_t partition_size, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream);

pa_status_t paged_attention_decode_reduce(void* out, const int32_t* context_lens, int32_t max_blocks_per_seq,
                                          int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                                          int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                          pa_dtype_t q_dtype, pa_dtype_t kv_dtype, int32_t partition_size,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_append -- one whole decode step in one pass: the slot mapping
 * and cache write of every sequence's newest token ("kernel 1") fused into the decode
 * attention ("kernel 2").  [CI BlockedKeyValueCache; CI KVCache Quant; CI PagedAttention]
 *
 * The newest token of sequence s sits at position L-1 (L = context_lens[s], which counts
 * it).  Its rows key[s], value[s] ([num_kv_heads][head_dim], q_dtype, dense, 16-byte
 * aligned) are stored at slot block_tables[s][(L-1)/B]*B + (L-1)%B of the pools (cast to
 * E5M2 when kv_dtype is FP8_E5M2, quantised to codes and a row scale when it is INT8 or
 * FP8_E4M3, exactly as kv_cache_write does), and the attention is paged_attention_decode over
 * all L tokens.  The result, pools and output, is bit-identical to paged_kv_slot_mapping +
 * kv_cache_write + paged_attention_decode with the same partition size.  A sequence with
 * L = 0 appends nothing.  A slot whose table entry is outside [0, num_blocks) is not
 * written.
 *
 * flags: PA_APPEND_SKIP_REDUCE -- run only the streaming pass; the caller then runs
 *        paged_attention_decode_reduce (same arguments) when a sequence is split.
 *        Without it the reduce kernel is launched after the streaming pass.
 */
#define PA_APPEND_SKIP_REDUCE 1

pa_status_t paged_attention_decode_append(void* out, const void* query, const void* key, const void* value,
                                          void* key_cache, void* value_cache, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                          int32_t max_context_len, float scale, pa_dtype_t q_dtype,
                                          pa_dtype_t kv_dtype, int32_t partition_size, int32_t flags,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_varlen -- one continuous-batching step: prefill chunks and decode tokens
 * packed into one 1-D token stream without padding.  [CI Continuous Batching: prefill and
 * decode are kept apart but no padding is added, the operators take 1-D input; OPT 2.3.2:
 * prefill is GEMM-bound, decode GEMV-bound]
 *
 * Sequence s owns query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1: its n_s newest tokens,
 * whose K/V rows must already be in the cache (kv_cache_write first).  Its context holds
 * L = context_lens[s] tokens, the new ones included, so query row i of the sequence sits at
 * position L - n_s + i.  With causal = 1 it attends keys 0 .. L-n_s+i (the mask aligned to
 * the end of the context); with causal = 0 every query row attends all L keys.
 *   out, query    [total_q][num_kv_heads*gqa_group][head_dim], bf16
 *   cu_seqlens_q  int32 [num_seqs + 1], non-decreasing, cu_seqlens_q[0] = 0,
 *                 cu_seqlens_q[num_seqs] = total_q; max_q_len >= every n_s
 *   other arguments as in paged_attention_decode; the workspace is sized by
 *   paged_attention_workspace_size(num_seqs, ...) and serves the 1-token rows.
 * Rows with n_s = 1 go through the decode kernels (split-KV when partition_size asks for
 * it); rows of sequences with n_s >= 2 through MFMA: when max_q_len * gqa_group <= 32 (a few
 * tokens per sequence, e.g. draft tokens of speculative decoding) one pass over each context
 * serves all its rows, otherwise 128-row query tiles.  When total_q = num_seqs * max_q_len and
 * max_q_len >= 2 no sequence has a single row and the decode kernel is not launched; when
 * max_q_len <= 1 only the decode kernel is.
 * Supported: bf16 query; bf16 or FP8_E5M2 cache (E5M2 codes widen exactly to f16, and the
 * multi-token rows then run on the f16 MFMA with the query and the probabilities in f16; the
 * query range is then that of paged_attention_decode over 8-bit caches: below 65536 in
 * magnitude, a larger element leaving its own row and head unspecified).  A row
 * whose position is negative (n_s > L) sees no key and comes out zero.
 */
pa_status_t paged_attention_varlen(void* out, const void* query, const void* key_cache, const void* value_cache,
                                   const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                                   int32_t total_q, int32_t max_q_len, int32_t num_kv_heads, int32_t gqa_group,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                                   float scale, int32_t causal, pa_dtype_t q_dtype, pa_dtype_t kv_dtype,
                                   int32_t partition_size, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * ---------------------------------------------------------------------------------------
 * Block manager (host side): which physical blocks of the pool each sequence owns.
 * [CI BlockedKeyValueCache: blocks are taken from the pool as tokens arrive, and only a
 *  sequence's last block is partly empty; OPT 2.1.2: a pool of blocks reserved up front, a
 *  table from logical to physical blocks, several logical blocks may name one physical block,
 *  a block in use has a reference count of one or more and is freed when it drops to zero;
 *  TACO Prefix Cache: the cache of earlier prompts is kept as a prefix tree, and the matching
 *  part of a new prompt is read from it instead of being computed]
 *
 * Rules (the pages fix the reference counting; the rest is this library's choice):
 *   - A new block is the lowest-numbered free block.
 *   - A sequence given its token ids registers each block it fills completely in the prefix
 *     tree, keyed by (parent block, the block's block_size token ids); the first block's
 *     parent is "none".  The caller must write a registered block's K/V before any later call
 *     can hand the block to another sequence (in one serving step: write, then schedule).
 *   - pa_bm_add_sequence with token ids reuses the longest chain of registered blocks that
 *     matches the prompt, up to (num_tokens - 1) / block_size blocks so that at least one token
 *     is left to compute; *cached_tokens tells how many leading tokens are already stored.
 *   - A block whose count drops to zero is free again if it is not registered; a registered
 *     one stays reusable until its block is needed: then the least recently released
 *     registered block with no registered child is evicted (ties: deeper first, then lower id).
 *   - Copy on write: appending to a sequence whose last, partly filled block is shared moves the
 *     sequence to a new block and reports the copy (old -> new) for paged_kv_copy_blocks.
 *   - Every call either succeeds or changes nothing.  PA_ERR_OUT_OF_BLOCKS: the pool (free plus
 *     evictable blocks) cannot supply the blocks the call needs.
 * A manager is not thread-safe; different managers may be used from different threads.
 * ---------------------------------------------------------------------------------------
 */
typedef struct pa_block_manager pa_block_manager;

/* A manager for a pool of num_blocks blocks of block_size tokens (both > 0). */
pa_status_t pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** manager);
void pa_bm_destroy(pa_block_manager* manager);

/*
 * A new sequence seq_id (not in use) holding num_tokens >= 0 tokens.  token_ids (host,
 * [num_tokens]) may be null: then the sequence takes no part in prefix reuse, and its appends
 * must pass null too.  *cached_tokens (may be null) = leading tokens whose K/V are already in
 * reused blocks (a multiple of block_size); the caller writes the rest.
 */
pa_status_t pa_bm_add_sequence(pa_block_manager* manager, int64_t seq_id, const int32_t* token_ids,
                               int32_t num_tokens, int32_t* cached_tokens);

/*
 * Append num_tokens >= 0 tokens to seq_id (token_ids as for pa_bm_add_sequence).  When the
 * last block is partly filled and shared, the sequence moves to a new block first and the copy
 * is reported as copies[0] = old block, copies[1] = new block, *num_copies = 1 (0 otherwise);
 * copies must then hold max_copies >= 1 pairs.
 */
pa_status_t pa_bm_append(pa_block_manager* manager, int64_t seq_id, const int32_t* token_ids, int32_t num_tokens,
                         int32_t* copies, int32_t max_copies, int32_t* num_copies);

/* child_id (not in use) shares every block of parent_id (counts + 1): a fork of the sequence. */
pa_status_t pa_bm_fork(pa_block_manager* manager, int64_t parent_id, int64_t child_id);

/* Release every block of seq_id and forget the sequence. */
pa_status_t pa_bm_free_sequence(pa_block_manager* manager, int64_t seq_id);

/*
 * The block table of seq_id: table[0 .. *num_blocks-1] (host, max_blocks entries), and its
 * token count.  PA_ERR_INVALID_ARGUMENT if it does not fit in max_blocks.
 */
pa_status_t pa_bm_block_table(const pa_block_manager* manager, int64_t seq_id, int32_t* table, int32_t max_blocks,
                              int32_t* num_blocks, int32_t* num_tokens);

/*
 * Pool state: free (never registered or released unregistered) blocks, registered blocks
 * (held or evictable), blocks with a count of one or more.  Any pointer may be null.
 */
pa_status_t pa_bm_stats(const pa_block_manager* manager, int32_t* free_blocks, int32_t* registered_blocks,
                        int32_t* used_blocks);

/*
 * paged_kv_copy_blocks -- copy whole blocks of both pools: for i < num_pairs, block
 * pairs[2i] -> block pairs[2i+1] (every KV head, every slot).  Carries out the copies that
 * pa_bm_append reports.  pairs: device int32 [2 * num_pairs]; a pair with an entry outside
 * [0, num_blocks) or src == dst is skipped; two pairs with the same destination race.
 * cache_dtype: any pool type (bytes are copied; an INT8 or FP8_E4M3 key block carries both rows'
 * scales).
 */
pa_status_t paged_kv_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int32_t num_pairs,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 pa_dtype_t cache_dtype, hipStream_t stream);

/*
 * ---------------------------------------------------------------------------------------
 * Step scheduler (host side): which sequences run in each step, for continuous batching.
 * [CI Continuous Batching: prefill and decode are computed apart, without padding, and a
 *  prefill step runs when the inputs waiting for prefill reach a set ratio, so that most
 *  steps are fast decode steps; OPT 2.4, Continuous Batching: step-level scheduling over a
 *  Running and a Waiting queue, a finished sequence leaves Running and a waiting one takes its
 *  place; OPT 2.4, Dynamic Batching: after every step the Running queue grows or shrinks with
 *  the free memory; OPT 2.1.2: block-granular accounting tells how many more blocks fit (no
 *  overflow), and max_num_batch_tokens bounds the tokens of one batch]
 *
 * A request is a prompt of token ids and a budget of new tokens.  Waiting is a FIFO of
 * requests holding no blocks; Running holds the admitted sequences (in admission order), all
 * of whose K/V except their newest token are in the cache.  Each pa_sched_step makes one step:
 *   - Prefill step, when Waiting is not empty, Running has room (< max_running) and either
 *     Running is empty or |Waiting| >= prefill_ratio * |Running|: requests are admitted from
 *     the head of Waiting, in order, while Running has room, the step's known-token total
 *     stays within max_batch_tokens (the first admitted request always fits, see add) and the
 *     block manager can hold the sequence (pa_bm_add_sequence with its token ids, so a cached
 *     prefix is reused).  The first request that does not fit ends admission.  Each admitted
 *     sequence's query rows are its tokens past the reused prefix.  If nothing is admitted the
 *     step is a decode step instead.
 *   - Decode step: every running sequence, in admission order, appends its newest token
 *     (pa_bm_append; a copy on write is reported in copies) and has it as its one query row.
 *     When the pool cannot supply a block, the most recently admitted running sequence is
 *     preempted (its blocks released, its known tokens -- prompt and generated -- put back at
 *     the head of Waiting, to be prefilled again), until the append succeeds or the appending
 *     sequence itself was preempted.
 *   - Idle step (kind PA_STEP_IDLE): nothing to run.
 * pa_sched_commit then takes, for every sequence of that step's batch in its order, the token
 * it produced and whether it finished (for instance an end-of-sequence token).  A sequence
 * also finishes when it has produced max_new_tokens tokens.  Finished sequences release their
 * blocks (prefix-registered blocks stay cached) and leave Running.  A step must be committed
 * before the next one (PA_ERR_INVALID_ARGUMENT otherwise); a step with no sequences needs no
 * commit.
 * The manager passed at creation is used only by the scheduler while it exists (sequence ids
 * are the request ids).  Not thread-safe.
 * ---------------------------------------------------------------------------------------
 */
typedef struct pa_scheduler pa_scheduler;

typedef struct {
  int32_t max_running;         /* most sequences in Running (> 0) */
  int32_t max_batch_tokens;    /* most known tokens admitted by one prefill step (> 0) */
  float prefill_ratio;         /* > 0, finite */
  int32_t max_blocks_per_seq;  /* width of the block tables a step fills (> 0) */
} pa_sched_config;

#define PA_STEP_IDLE 0
#define PA_STEP_PREFILL 1
#define PA_STEP_DECODE 2

/*
 * One step's batch, in host arrays the caller owns.  Capacities (set by the caller, checked
 * before anything changes): seq_ids, context_lens: max_running entries; cu_seqlens_q:
 * max_running + 1; block_tables: max_running * max_blocks_per_seq (row-major, -1 past each
 * sequence's blocks); input_tokens: max(max_batch_tokens, max_running); copies: 2 *
 * max_running; preempted: max_running.  Outputs feed paged_kv_slot_mapping (cu_tokens =
 * cu_seqlens_q, end_pos = context_lens), kv_cache_write and paged_attention_varlen (decode
 * steps may also use paged_attention_decode), after paged_kv_copy_blocks of the copies.
 */
typedef struct {
  int64_t* seq_ids;
  int32_t* cu_seqlens_q;
  int32_t* context_lens;
  int32_t* block_tables;
  int32_t* input_tokens;  /* token id of every query row, packed like the rows */
  int32_t* copies;        /* (src, dst) block pairs */
  int64_t* preempted;     /* requests moved back to Waiting during this step */
  int32_t kind;           /* PA_STEP_* */
  int32_t num_seqs;
  int32_t total_q;
  int32_t max_q_len;
  int32_t max_context_len;
  int32_t num_copies;
  int32_t num_preempted;
} pa_sched_batch;

/* A scheduler over `manager` (which must outlive it) with the given limits. */
pa_status_t pa_sched_create(const pa_sched_config* config, pa_block_manager* manager, pa_scheduler** scheduler);
void pa_sched_destroy(pa_scheduler* scheduler);

/*
 * Queue a request at the tail of Waiting: request_id (not in use), prompt (host, prompt_len
 * >= 1 token ids), max_new_tokens >= 1.  prompt_len + max_new_tokens - 1 (the most tokens a
 * prefill of this request can carry, after a preemption) must be at most max_batch_tokens and
 * fit max_blocks_per_seq blocks (PA_ERR_UNSUPPORTED otherwise).
 */
pa_status_t pa_sched_add_request(pa_scheduler* scheduler, int64_t request_id, const int32_t* prompt,
                                 int32_t prompt_len, int32_t max_new_tokens);

/* Make the next step (see above) and describe it in *batch. */
pa_status_t pa_sched_step(pa_scheduler* scheduler, pa_sched_batch* batch);

/*
 * Results of the last step: next_tokens[i] and finished[i] (0 or 1; may be null: none
 * finished early) for the i-th sequence of its batch, num_seqs entries.
 */
pa_status_t pa_sched_commit(pa_scheduler* scheduler, const int32_t* next_tokens, const uint8_t* finished,
                            int32_t num_seqs);

/* Requests waiting, sequences running, requests finished and preemptions so far.  Any pointer
 * may be null. */
pa_status_t pa_sched_stats(const pa_scheduler* scheduler, int32_t* waiting, int32_t* running, int64_t* finished,
                           int64_t* preemptions);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
