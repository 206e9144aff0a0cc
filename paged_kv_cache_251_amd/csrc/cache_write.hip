// Slot mapping and the cache write ("kernel 1") for gfx950.
//
// Colossal-Inference release post, "分块式KV缓存 (BlockedKeyValueCache)": logical blocks map
// through a block table to physical blocks anywhere in the pool; "KV缓存量化 (KVCache
// Quant)": the kernel that stores new keys and values casts them to FP8 E5M2 on the way.
// LLM inference frameworks overview, "LMDeploy": an INT8 KV cache; LLM inference optimisation
// overview, 2.6: low-bit caches.  The schemes (INT8 codes or FP8 E4M3 codes, one float32 scale
// per (token, KV head) row) are this library's.
#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {

// One thread per packed token row: find its sequence by binary search over cu, then
// slot = table[p / B] * B + p % B for its logical position p.
__global__ __launch_bounds__(256) void slot_mapping_kernel(int32_t* __restrict__ slots,
                                                           const int32_t* __restrict__ cu,
                                                           const int32_t* __restrict__ end_pos,
                                                           const int32_t* __restrict__ tables,
                                                           int32_t max_blocks, int32_t num_seqs,
                                                           int32_t num_tokens, int32_t block_size,
                                                           int32_t num_blocks) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  int lo = 0, hi = num_seqs;  // invariant: the answer is in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int a = cu[s], b = cu[s + 1];
  int slot = -1;
  if (t >= a && t < b) {
    const int pos = end_pos[s] - (b - a) + (t - a);
    const int lb = pos >= 0 ? pos / block_size : -1;
    if (lb >= 0 && lb < max_blocks) {
      const int phys = tables[(size_t)s * max_blocks + lb];
      if (phys >= 0 && phys < num_blocks) slot = phys * block_size + pos % block_size;
    }
  }
  slots[t] = slot;
}

hipError_t launch_slot_mapping(int32_t* slots, const int32_t* cu, const int32_t* end_pos,
                               const int32_t* tables, int32_t max_blocks, int32_t num_seqs,
                               int32_t num_tokens, int32_t block_size, int32_t num_blocks,
                               hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int blocks = (num_tokens + 255) / 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks), dim3(256), 0, stream, slots, cu, end_pos, tables,
                     max_blocks, num_seqs, num_tokens, block_size, num_blocks);
  return hipGetLastError();
}

// One thread per 16 source bytes of a row (4 f32 or 8 bf16 elements).  Source rows are
// [token][kv_head][D]; destination [block][kv_head][B][D].
template <int SRC, int DST>
__global__ __launch_bounds__(256) void cache_write_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                                                          uint8_t* __restrict__ key_cache,
                                                          uint8_t* __restrict__ value_cache,
                                                          const int32_t* __restrict__ slots, int32_t num_tokens,
                                                          int32_t num_kv_heads, int32_t head_dim,
                                                          int32_t block_size, int32_t num_blocks) {
  constexpr int SRC_SZ = KvBytes<SRC>::value;
  constexpr int EPC = 16 / SRC_SZ;  // elements per chunk
  const int chunks_per_row = num_kv_heads * head_dim / EPC;
  const size_t total = (size_t)num_tokens * chunks_per_row;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int t = (int)(i / chunks_per_row);
  const int c = (int)(i % chunks_per_row);
  const int slot = slots[t];
  if (slot < 0 || slot >= num_blocks * block_size) return;
  const int h = (c * EPC) / head_dim;
  const int d = (c * EPC) % head_dim;
  const size_t dst_elem = (((size_t)(slot / block_size) * num_kv_heads + h) * block_size + slot % block_size) *
                              head_dim + d;
  const uint4 kin = key[i];
  const uint4 vin = value[i];
  if constexpr (SRC == DST) {
    *reinterpret_cast<uint4*>(key_cache + dst_elem * SRC_SZ) = kin;
    *reinterpret_cast<uint4*>(value_cache + dst_elem * SRC_SZ) = vin;
  } else {  // bf16 -> E5M2, 8 elements -> 8 bytes
    auto cast8 = [](uint4 w) {
      const uint32_t c0 = bf16_to_e5m2(w.x & 0xFFFFu) | (bf16_to_e5m2(w.x >> 16) << 8) |
                          (bf16_to_e5m2(w.y & 0xFFFFu) << 16) | (bf16_to_e5m2(w.y >> 16) << 24);
      const uint32_t c1 = bf16_to_e5m2(w.z & 0xFFFFu) | (bf16_to_e5m2(w.z >> 16) << 8) |
                          (bf16_to_e5m2(w.w & 0xFFFFu) << 16) | (bf16_to_e5m2(w.w >> 16) << 24);
      return make_uint2(c0, c1);
    };
    *reinterpret_cast<uint2*>(key_cache + dst_elem) = cast8(kin);
    *reinterpret_cast<uint2*>(value_cache + dst_elem) = cast8(vin);
  }
}

// bf16 rows -> scaled 8-bit pool (KV_I8: codes in [-127, 127], scale amax / 127; KV_E4M3: FP8
// E4M3 codes of x * 448 / amax, scale amax / 448).  D/8 consecutive lanes take one (token, KV
// head) row, 8 elements each (one 16-byte load); the row's amax is reduced across them, then
// every lane stores its 8 codes and the row's first lane the scale.  The maximum is taken on
// the bf16 magnitude patterns as integers (order-preserving for non-NaN values; NaN mapped
// below every number), so NaN elements are ignored whatever their payload and an all-NaN row
// gets a NaN amax.
template <int D, int KV>
__global__ __launch_bounds__(256) void cache_write_q8_kernel(const uint4* __restrict__ key,
                                                             const uint4* __restrict__ value,
                                                             uint8_t* __restrict__ key_cache,
                                                             uint8_t* __restrict__ value_cache,
                                                             const int32_t* __restrict__ slots, int32_t num_tokens,
                                                             int32_t num_kv_heads, int32_t num_blocks) {
  constexpr int LPR = D / 8;  // lanes per row; divides 64, so a row never straddles waves
  constexpr int KTILE = KTileStride<KV, D>::value, VTILE = VTileStride<KV, D>::value;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)num_tokens * num_kv_heads * LPR;
  if (i >= total) return;  // total is a multiple of LPR: a row's lanes leave together
  const size_t row = i / LPR;
  const int c = (int)(i % LPR);
  const int t = (int)(row / num_kv_heads), h = (int)(row % num_kv_heads);
  const int slot = slots[t];
  if (slot < 0 || slot >= num_blocks * 16) return;  // same slot on every lane of the row
  const int r = slot & 15;
  const size_t unit = (size_t)(slot >> 4) * num_kv_heads + h;
  const size_t ktile = unit * KTILE;  // holds the key codes, then the key and the value scales

  auto quantize = [&](uint4 w, uint8_t* codes, float* scale) {
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
    float x[8];
    int key_max = -1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16lo(words[k]);
      x[2 * k + 1] = bf16hi(words[k]);
      key_max = max(key_max, max(bf16_mag_key(words[k]), bf16_mag_key(words[k] >> 16)));
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) key_max = max(key_max, __shfl_xor(key_max, off));
    const float amax = q8_amax(key_max);
    const float inv = q8_inv<KV>(amax);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) packed[k >> 2] |= q8_code<KV>(x[k], inv) << (8 * (k & 3));
    *reinterpret_cast<uint2*>(codes + (size_t)r * D + (size_t)c * 8) = make_uint2(packed[0], packed[1]);
    if (c == 0) *scale = amax / Q8Range<KV>::value;
  };
  float* kscale = reinterpret_cast<float*>(key_cache + ktile + q8_scale_offset<D>(r));
  quantize(key[i], key_cache + ktile, kscale);
  quantize(value[i], value_cache + unit * VTILE, kscale + kValueScaleOffset / 4);
}

hipError_t launch_cache_write(const void* key, const void* value, void* key_cache, void* value_cache,
                              const int32_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks, int src_kind,
                              int cache_kind, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int src_sz = src_kind == KV_F32 ? 4 : 2;
  const size_t total = (size_t)num_tokens * num_kv_heads * head_dim * src_sz / 16;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  auto k = reinterpret_cast<const uint4*>(key);
  auto v = reinterpret_cast<const uint4*>(value);
  auto kc = reinterpret_cast<uint8_t*>(key_cache);
  auto vc = reinterpret_cast<uint8_t*>(value_cache);
  if (src_kind == KV_F32 && cache_kind == KV_F32)
    hipLaunchKernelGGL((cache_write_kernel<KV_F32, KV_F32>), dim3(blocks), dim3(256), 0, stream, k, v, kc, vc, slots,
                       num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
  else if (src_kind == KV_BF16 && cache_kind == KV_BF16)
    hipLaunchKernelGGL((cache_write_kernel<KV_BF16, KV_BF16>), dim3(blocks), dim3(256), 0, stream, k, v, kc, vc,
                       slots, num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
  else if (src_kind == KV_BF16 && cache_kind == KV_E5M2)
    hipLaunchKernelGGL((cache_write_kernel<KV_BF16, KV_E5M2>), dim3(blocks), dim3(256), 0, stream, k, v, kc, vc,
                       slots, num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
  else if (src_kind == KV_BF16 && cache_kind == KV_I8 && block_size == 16 && head_dim == 128)
    hipLaunchKernelGGL((cache_write_q8_kernel<128, KV_I8>), dim3(blocks), dim3(256), 0, stream, k, v, kc, vc,
                       slots, num_tokens, num_kv_heads, num_blocks);
  else if (src_kind == KV_BF16 && cache_kind == KV_I8 && block_size == 16 && head_dim == 64)
    hipLaunchKernelGGL((cache_write_q8_kernel<64, KV_I8>), dim3(blocks), dim3(256), 0, stream, k, v, kc, vc,
                       slots, num_tokens, num_kv_heads, num_blocks);
  else if (src_kind == KV_BF16 && cache_kind == KV_E4M3 && block_size == 16 && head_dim == 128)
    hipLaunchKernelGGL((cache_write_q8_kernel<128, KV_E4M3>), dim3(blocks), dim3(256), 0, stream, k, v, kc, vc,
                       slots, num_tokens, num_kv_heads, num_blocks);
  else if (src_kind == KV_BF16 && cache_kind == KV_E4M3 && block_size == 16 && head_dim == 64)
    hipLaunchKernelGGL((cache_write_q8_kernel<64, KV_E4M3>), dim3(blocks), dim3(256), 0, stream, k, v, kc, vc,
                       slots, num_tokens, num_kv_heads, num_blocks);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Whole-block copies of both pools (copy on write of a shared, partly filled block): work-group
// (pair, pool) copies one block of `block_bytes` with 16-byte loads and stores.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* key_cache, uint8_t* value_cache,
                                                          const int32_t* pairs, size_t k_block_bytes,
                                                          size_t v_block_bytes, int32_t num_blocks) {
  const int32_t src = pairs[2 * (size_t)blockIdx.x], dst = pairs[2 * (size_t)blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  uint8_t* base = blockIdx.y == 0 ? key_cache : value_cache;
  const size_t block_bytes = blockIdx.y == 0 ? k_block_bytes : v_block_bytes;
  const uint4* from = reinterpret_cast<const uint4*>(base + (size_t)src * block_bytes);
  uint4* to = reinterpret_cast<uint4*>(base + (size_t)dst * block_bytes);
  for (size_t i = threadIdx.x; i < block_bytes / 16; i += 256) to[i] = from[i];
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int32_t num_pairs,
                              size_t k_block_bytes, size_t v_block_bytes, int32_t num_blocks, hipStream_t stream) {
  if (num_pairs <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, stream,
                     static_cast<uint8_t*>(key_cache), static_cast<uint8_t*>(value_cache), pairs, k_block_bytes,
                     v_block_bytes, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
