// One launch for a packed (varlen) step that holds both prefill chunks and decode tokens.
//
// The release post's continuous batching (Colossal-Inference, "连续批量化算法 (Continuous
// Batching)") keeps prefill and decode tokens in one unpadded 1-D batch; the optimisation
// overview (2.3.2 "高性能算子") notes that prefill is GEMM-bound and decode GEMV-bound, so the two
// use different parts of the chip: the matrix cores, and the memory system.  Run back to back,
// each leaves the other's part idle.  Here one grid carries both roles: work-group i is either a
// prefill unit (a 128-row query tile of one KV head, on MFMA; prefill_body.hpp) or a decode unit
// (one (sequence, KV head) context streamed whole; decode_body.hpp), the roles interleaved evenly
// in dispatch order, each list longest first.  A CU then holds work-groups of both roles at once:
// while one waits on HBM the other keeps the matrix cores busy.
//
// Work-group i runs on XCD i % 8 (round-robin dispatch), and every XCD has its own L2.  The query
// tiles of one (sequence, KV head) re-read the same K/V tiles, so the interleave is made within
// each residue class of the dispatch index mod 8, and the unit of rank r goes to class r % 8: with
// up to 8 KV heads (or a multiple of 8) every unit of a head runs on the same XCD and finds its
// tiles in that XCD's L2.
//
// The decode role runs only whole-context passes (no split-KV partitions; the caller's launch
// falls back to the two kernels otherwise).
#include "decode_body.hpp"
#include "pa_device.hpp"
#include "pa_launch.hpp"
#include "prefill_body.hpp"

namespace pa {

// LDS of a two-role work-group: the larger of the two roles' needs.
template <int D, int G>
struct PackedSmem {
  static constexpr int DEC = DecodeSmem<G, D, 4>::BYTES;
  static constexpr int PRE = PrefillSmem<D>::BYTES;
  static constexpr int BYTES = DEC > PRE ? DEC : PRE;
};

// Position i of the dispatch order holds a prefill work-group when floor((i+1) n_pre / total) >
// floor(i n_pre / total): the n_pre prefill work-groups are spread evenly over the total.
__device__ __forceinline__ int2 packed_role(int i, int n_pre, int total) {
  const long long before = (long long)i * n_pre / total;
  const long long upto = (long long)(i + 1) * n_pre / total;
  return upto > before ? make_int2(1, (int)before) : make_int2(0, i - (int)before);
}

// Prefill work-groups the batch really needs: ceil(n_s / TOKW) query tiles of every sequence with
// n_s >= 2 rows, per KV head (the host only knows an upper bound).  Wave 0 counts, every wave reads.
template <int TOKW>
__device__ __forceinline__ int packed_prefill_units(const DecodeParams& p, int num_seqs, int* sm) {
  if (threadIdx.x < 64) {
    int c = 0;
    for (int s = threadIdx.x; s < num_seqs; s += 64) {
      const int n = load_invariant(p.cu_q + s + 1) - load_invariant(p.cu_q + s);
      c += n >= 2 ? (n + TOKW - 1) / TOKW : 0;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
    if (threadIdx.x == 0) *sm = c * p.num_kv_heads;
  }
  __syncthreads();
  const int u = *sm;
  __syncthreads();  // the slot is reused by the roles' own LDS
  return u;
}

template <int D, int G, bool E8>
__global__ __launch_bounds__(256, 2) void packed_step_kernel(const DecodeParams p, int n_pre_bound, int n_dec) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[PackedSmem<D, G>::BYTES];
  // The roles are interleaved over the prefill work-groups the batch needs, not the host's bound;
  // each class's surplus positions come last in it and return at once.
  const int n_pre =
      min(n_pre_bound, packed_prefill_units<128 / G>(p, n_dec / p.num_kv_heads, reinterpret_cast<int*>(smem)));
  const int x = (int)blockIdx.x & 7, q = (int)blockIdx.x >> 3;  // class and position in it
  const int npx = n_pre > x ? (n_pre - x + 7) >> 3 : 0;          // ranks x, x + 8, ... of each list
  const int ndx = n_dec > x ? (n_dec - x + 7) >> 3 : 0;
  if (q >= npx + ndx) return;
  const int2 r = packed_role(q, npx, npx + ndx);
  const int rank = r.y * 8 + x;
  if (r.x) {
    prefill_body<D, G, E8>(p, rank, 0, 0, 1, reinterpret_cast<uint16_t*>(smem));
  } else {
    constexpr int KV = E8 ? KV_E5M2 : KV_BF16;
    int* sm_i = reinterpret_cast<int*>(smem);
    float* sm_f = reinterpret_cast<float*>(smem + 4 * DecodeSmem<G, D, 4>::INTS);
    decode_body<KV, D, G, 4>(p, rank % p.num_kv_heads, 0, rank / p.num_kv_heads, p.num_kv_heads,
                             n_dec / p.num_kv_heads, sm_i, sm_f);
  }
}

template <int D, int G, bool E8>
static hipError_t launch_packed_dg(const DecodeParams& p, int num_seqs, int total_q, int max_q_len,
                                   hipStream_t stream) {
  constexpr int TOKW = 128 / G;
  DecodeParams q = p;
  // prefill work-groups: as many as the longest-first schedule can hand units to (see the
  // prefill kernel's launcher); the spare ones return at once
  const long long tiles_per_seq = (max_q_len + TOKW - 1) / TOKW;
  const long long chunks = std::min<long long>(num_seqs, total_q / 2);
  const long long units = std::min<long long>((total_q + chunks * (TOKW - 1)) / TOKW, tiles_per_seq * num_seqs);
  const long long n_pre = units * p.num_kv_heads;
  const long long n_dec = (long long)num_seqs * p.num_kv_heads;
  // eight classes of ceil(n_pre / 8) + ceil(n_dec / 8) positions
  const long long grid = 8 * ((n_pre + 7) / 8 + (n_dec + 7) / 8);
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  q.sched_seqs = num_seqs;
  q.longest_first = 1;
  q.snake = 0;
  q.resident = 0;
  hipLaunchKernelGGL((packed_step_kernel<D, G, E8>), dim3((unsigned)grid), dim3(256), 0, stream, q, (int)n_pre,
                     (int)n_dec);
  return hipGetLastError();
}

template <int D, bool E8>
static hipError_t launch_packed_d(const DecodeParams& p, int gqa, int num_seqs, int total_q, int max_q_len,
                                  hipStream_t stream) {
  switch (gqa) {
    case 1: return launch_packed_dg<D, 1, E8>(p, num_seqs, total_q, max_q_len, stream);
    case 2: return launch_packed_dg<D, 2, E8>(p, num_seqs, total_q, max_q_len, stream);
    case 4: return launch_packed_dg<D, 4, E8>(p, num_seqs, total_q, max_q_len, stream);
    case 8: return launch_packed_dg<D, 8, E8>(p, num_seqs, total_q, max_q_len, stream);
    case 16: return launch_packed_dg<D, 16, E8>(p, num_seqs, total_q, max_q_len, stream);
  }
  return hipErrorInvalidValue;
}

// Every work-group of the two-role kernel ranks the batch's sequences (O(n^2 / threads) each), so
// large batches take the two kernels back to back instead.  Measured with 4 prefill chunks (32
// query / 8 KV heads): one launch 241.8 against 300.4 us with 128 decode rows, 408.3 against 463.7
// with 252, but 894.9 against 799.6 with 508.
constexpr int kPackedMaxSeqs = 256;

bool packed_step_applies(const DecodeParams& p, int num_seqs, int max_q_len) {
  return p.max_parts <= 1 && num_seqs <= kPackedMaxSeqs && num_seqs <= kMaxScheduledSeqs &&
         num_seqs <= kMaxRankedSeqs && max_q_len >= 2;
}

hipError_t launch_packed_step(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs, int total_q,
                              int max_q_len, hipStream_t stream) {
  const bool e8 = kv_kind == KV_E5M2;
  if (!e8 && kv_kind != KV_BF16) return hipErrorInvalidValue;
  if (head_dim == 128)
    return e8 ? launch_packed_d<128, true>(p, gqa, num_seqs, total_q, max_q_len, stream)
              : launch_packed_d<128, false>(p, gqa, num_seqs, total_q, max_q_len, stream);
  if (head_dim == 64)
    return e8 ? launch_packed_d<64, true>(p, gqa, num_seqs, total_q, max_q_len, stream)
              : launch_packed_d<64, false>(p, gqa, num_seqs, total_q, max_q_len, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
