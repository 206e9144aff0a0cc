// Paged decode attention for gfx950: one work-group per (partition, KV head, sequence).
//
// What is computed (Colossal-Inference release post, "分页注意力算法 (PagedAttention)":
// decode attention is a memory-bound GEMV over the cached keys and values, read block by
// block through the block table; LLM inference optimisation overview, 2.2.2 "GQA": the
// query heads of a group share one KV head; 2.2.1 "Flash Attention": softmax reduced
// without the whole input, which is what lets a context be split into partitions):
//   out[s][h] = sum_t 2^(S_t - M) V[t][g] / sum_t 2^(S_t - M),  S_t = scale*log2(e) q[s][h].K[t][g]
//
// Mapping onto CDNA4 (wave64):
//  * A KV tile (one physical block, one KV head) is block_size x head_dim contiguous
//    elements.  A wave reads it with 4 coalesced loads; in each, 16-lane row r holds
//    token 4i + r and lane c of the row holds head_dim/16 consecutive elements.
//  * All G query heads of the group are kept in registers of every lane (only the
//    lane's head_dim/16 slice), in a lane-dependent order that lets one pass of 4 DPP
//    steps both finish the dot products and leave head h's score on lanes
//    h*16/G .. h*16/G + 16/G - 1 of the row (row_reduce_heads).
//  * Softmax state is kept per 16-lane row (its own tokens), so the loop needs no
//    cross-row traffic.  The running max is only raised when a block's max exceeds it
//    by more than TAU (2^8): exact, since the same stale max is used for the numerator
//    and the denominator, and it makes the rescale branch rare.
//  * Probabilities reach the PV lanes by DPP row broadcast; V is accumulated in fp32
//    (f32 / bf16 caches) or with f16 dot2 over token pairs (E5M2, INT8 and E4M3 caches, whose
//    codes widen exactly to f16).  An INT8 or E4M3 key tile ends in its 16 key scales and then
//    the 16 value scales of the same tokens, each group ordered so that one 16-byte load gives a
//    lane the scales of its row's four tokens: the key scale multiplies the finished dot
//    product, the value scale the probability (in f16).
//  * Rows, then waves, are merged at the end; a single partition writes the output,
//    several write (o/l, m, l) to the workspace for the reduce kernel.
#include <atomic>
#include <mutex>

#include "decode_body.hpp"
#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {

template <int KV, int D, int G, int W>
__global__ __launch_bounds__(64 * W) void decode_partition_kernel(
    const DecodeParams p) {
  __shared__ int sm_i[DecodeSmem<G, D, W>::INTS];
  __shared__ float sm_f[DecodeSmem<G, D, W>::FLOATS];
  decode_body<KV, D, G, W>(p, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.x, gridDim.z, sm_i, sm_f);
}

// ---------------------------------------------------------------------------------------
// Waves per work-group of the partition kernel.  A whole-context pass (one work-group per
// (KV head, sequence)) takes 4: a CU holds two or more work-groups, so one that ends leaves the
// CU streaming for the others while the dispatcher refills it.  When the whole grid is resident
// at once, the snake order balances the sum of context lengths per CU; otherwise the plain
// longest-first order lets the dispatcher place the remaining, shorter contexts on whichever CU
// frees up first.  A split pass takes 1: each partition is streamed by one wave, whose merge of
// its four rows is the whole flush (no LDS merge across waves, no barrier), and a CU holds a
// dozen partitions at once; measured on 8 contexts of 32768 tokens in 512-token partitions, 3 to
// 4 % faster than four waves per partition.
// Groups of 8 or 16 query heads per KV head over a bf16 or E5M2 cache take the partition pass on
// MFMA (multiquery.hip).  With G = 8 the vector kernel spends twice the FMAs per KV byte of G = 4
// and falls behind the memory.  Measured on the fused decode step: 64 sequences of 512..2048
// tokens with 64 query / 8 KV heads 63.8 us against 69.5 us; 8 x 32768 tokens in 512-token
// partitions 187.5 us against 205.5 us for the partition launch.
#ifndef PA_DECODE_MFMA_WIDE_GROUPS
#define PA_DECODE_MFMA_WIDE_GROUPS 1
#endif
static_assert(kLongestFirstMaxSeqs <= kMaxRankedSeqs, "the ranking buffer holds every ranked sequence");

#ifndef PA_DECODE_WAVES_WHOLE
#define PA_DECODE_WAVES_WHOLE 4
#endif
#ifndef PA_DECODE_WAVES_SPLIT
#define PA_DECODE_WAVES_SPLIT 1
#endif

// CUs of the current device (cached per device).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int current_device_cus() { return device_cus(); }

// Work-groups of one instantiation of the decode kernel that one CU holds at once (cached per
// instantiation: every instantiation has the same function type, so the cache is keyed by the
// template arguments, not by the pointer's type).
template <int KV, int D, int G, int W>
static int resident_per_cu() {
  static std::atomic<int> cache{0};
  int c = cache.load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, decode_partition_kernel<KV, D, G, W>, 64 * W, 0) !=
          hipSuccess ||
      c <= 0)
    return 0;
  cache.store(c, std::memory_order_relaxed);
  return c;
}

template <int KV, int D, int G>
static hipError_t launch_parts_kv_d_g(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  // KV head fastest: consecutive work-groups go to different XCDs, and with 8 KV heads
  // each XCD streams one head of every sequence (equal shares whatever the lengths).
  dim3 grid(p.num_kv_heads, p.max_parts, num_seqs);
  if (p.max_parts <= 1) {
    constexpr int W = PA_DECODE_WAVES_WHOLE;
    auto kernel = decode_partition_kernel<KV, D, G, W>;
    DecodeParams q = p;
    q.snake = 0;
    q.resident = 0;
    if (p.longest_first) {  // the kernel applies the snake order when its units fit the resident grid
      const int cus = device_cus();
      const int per_cu = resident_per_cu<KV, D, G, W>();
      if (cus > 0 && per_cu > 0) {
        q.snake = cus;
        q.resident = cus * per_cu;
      }
      // a decode call (every sequence one row) whose units do not all fit: plain grid order, the
      // ranking would cost more than the order gains (packed batches: the kernel counts its rows)
      if (p.cu_q == nullptr && (long long)num_seqs * p.num_kv_heads > (long long)q.resident) q.longest_first = 0;
    }
    hipLaunchKernelGGL(kernel, grid, dim3(64 * W), 0, stream, q);
  } else {
    constexpr int W = PA_DECODE_WAVES_SPLIT;
    hipLaunchKernelGGL((decode_partition_kernel<KV, D, G, W>), grid, dim3(64 * W), 0, stream, p);
  }
  return hipGetLastError();
}

template <int KV, int D>
static hipError_t launch_parts_kv_d(const DecodeParams& p, int gqa, int num_seqs, hipStream_t stream) {
  switch (gqa) {
    case 1: return launch_parts_kv_d_g<KV, D, 1>(p, num_seqs, stream);
    case 2: return launch_parts_kv_d_g<KV, D, 2>(p, num_seqs, stream);
    case 4: return launch_parts_kv_d_g<KV, D, 4>(p, num_seqs, stream);
    case 8: return launch_parts_kv_d_g<KV, D, 8>(p, num_seqs, stream);
    case 16: return launch_parts_kv_d_g<KV, D, 16>(p, num_seqs, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_partitions(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs,
                                    hipStream_t stream) {
  if (PA_DECODE_MFMA_WIDE_GROUPS && decode_mfma_applies(p, kv_kind, head_dim, gqa))
    return launch_decode_mfma(p, kv_kind, head_dim, gqa, num_seqs, stream);
  if (head_dim == 128) {
    if (kv_kind == KV_F32) return launch_parts_kv_d<KV_F32, 128>(p, gqa, num_seqs, stream);
    if (kv_kind == KV_BF16) return launch_parts_kv_d<KV_BF16, 128>(p, gqa, num_seqs, stream);
    if (kv_kind == KV_E5M2) return launch_parts_kv_d<KV_E5M2, 128>(p, gqa, num_seqs, stream);
    if (kv_kind == KV_I8) return launch_parts_kv_d<KV_I8, 128>(p, gqa, num_seqs, stream);
    if (kv_kind == KV_E4M3) return launch_parts_kv_d<KV_E4M3, 128>(p, gqa, num_seqs, stream);
  } else if (head_dim == 64) {
    if (kv_kind == KV_F32) return launch_parts_kv_d<KV_F32, 64>(p, gqa, num_seqs, stream);
    if (kv_kind == KV_BF16) return launch_parts_kv_d<KV_BF16, 64>(p, gqa, num_seqs, stream);
    if (kv_kind == KV_E5M2) return launch_parts_kv_d<KV_E5M2, 64>(p, gqa, num_seqs, stream);
    if (kv_kind == KV_I8) return launch_parts_kv_d<KV_I8, 64>(p, gqa, num_seqs, stream);
    if (kv_kind == KV_E4M3) return launch_parts_kv_d<KV_E4M3, 64>(p, gqa, num_seqs, stream);
  }
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------------------------------
// Split-KV scratch of the entry point that allocates nothing: one array per GPU, held until the
// process ends.  In host code `scratch` is only a stand-in for the symbol, not a device address;
// the address of the current device's copy comes from hipGetSymbolAddress, taken once per device
// (with that device current) and kept.  The partition pass writes every partial the reduce pass
// reads in the same call, so nothing in it has to start at zero.
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace pa
