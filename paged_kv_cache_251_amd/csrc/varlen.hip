// Prefill part of a packed (varlen) step on gfx950 MFMA.
//
// A packed batch holds, per sequence, the n newest tokens of a context of L tokens
// (Colossal-Inference release post, "连续批量化算法 (Continuous Batching)": prefill and
// decode tokens go through the same 1-D operators without padding).  Their K/V rows are
// already in the cache.  Query token i of the sequence sits at position L-n+i and, when
// causal, sees keys 0..L-n+i (the mask aligned to the end of the context).  Sequences with
// n = 1 are decode rows and go through the decode kernel; this kernel takes n >= 2, where
// QK^T and PV are dense contractions (LLM inference optimisation overview, 2.3.2: prefill is
// GEMM-bound).
//
// Work-group = 4 waves = 128 query rows of one KV head: row r is (token i0 + r / G, head r % G),
// so the G heads that share the KV head share every K/V tile.  Each wave owns two 16-row
// tiles.  Per 64-key tile:
//   S^T[keys][rows] = K[keys][D] . Q^T[D][rows]     v_mfma_f32_16x16x32_bf16, A = K from LDS
//                                                    (row-major), B = Q from registers
//   O^T[D][rows]  += V^T[D][keys] . P^T[keys][rows]  A = V^T read from the row-major V tile
//                                                    with ds_read_b64_tr_b16, B = P straight
//                                                    from the S^T accumulators
// With S^T, lane l holds 4 consecutive keys of query row l%16 per 16-key tile; two tiles give
// the 8 keys the B operand of the PV step needs (keys 4j..4j+3 and 16+4j..16+4j+3 for lane
// group j = l/16), and V^T is read in the same key order, so P never goes through LDS.
// ds_read_b64_tr_b16 (checked on the device): within each 16-lane group, lane i's j-th 16-bit
// result is element i%4 of the 8 bytes read by lane 4j + i/4.  So if lane k of the group reads
// dims 4(k%4)..+3 of key k/4, lane i receives dim i of the 4 keys -- a column of V.
// Every accumulator of lane l belongs to row l%16: the online-softmax rescale is per lane.
//
// Order of work: a work unit is (sequence, 128-row query tile, KV head); the causal mask makes
// its cost proportional to the keys it sees, kv_end.  For batches of up to kMaxScheduledSeqs
// sequences the grid is one-dimensional and work-group j takes the unit of rank j / Hkv in
// descending kv_end over every sequence (head j % Hkv), so the dispatcher hands out the
// longest units first across all chunks, and the grid's spare work-groups come last.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "pa_device.hpp"
#include "pa_launch.hpp"
#include "prefill_body.hpp"

namespace pa {

template <int D, int G, bool E8>
__global__ __launch_bounds__(256, 2) void varlen_prefill_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[PrefillSmem<D>::ELEMS];
  prefill_body<D, G, E8>(p, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.y, lds);
}

template <int D, int G, bool E8>
static hipError_t launch_prefill_dg(const DecodeParams& p, int num_seqs, int total_q, int max_q_len,
                                   hipStream_t stream) {
  constexpr int TOKW = 128 / G;
  DecodeParams q = p;
  const long long tiles_per_seq = (max_q_len + TOKW - 1) / TOKW;
  if (num_seqs <= kMaxScheduledSeqs) {
    // At most min(N, total_q / 2) sequences have n >= 2, and together they hold at most
    // total_q tokens, so they have at most (total_q + that count * (TOKW - 1)) / TOKW tiles.
    const long long chunks = std::min<long long>(num_seqs, total_q / 2);
    const long long units = std::min<long long>((total_q + chunks * (TOKW - 1)) / TOKW, tiles_per_seq * num_seqs);
    q.sched_seqs = num_seqs;
    hipLaunchKernelGGL((varlen_prefill_kernel<D, G, E8>), dim3((unsigned)(units * p.num_kv_heads)), dim3(256), 0,
                       stream, q);
  } else {
    q.sched_seqs = 0;
    dim3 grid(p.num_kv_heads, (unsigned)tiles_per_seq, num_seqs);
    hipLaunchKernelGGL((varlen_prefill_kernel<D, G, E8>), grid, dim3(256), 0, stream, q);
  }
  return hipGetLastError();
}

template <int D, bool E8>
static hipError_t launch_prefill_d(const DecodeParams& p, int gqa, int num_seqs, int total_q, int max_q_len,
                                   hipStream_t stream) {
  switch (gqa) {
    case 1: return launch_prefill_dg<D, 1, E8>(p, num_seqs, total_q, max_q_len, stream);
    case 2: return launch_prefill_dg<D, 2, E8>(p, num_seqs, total_q, max_q_len, stream);
    case 4: return launch_prefill_dg<D, 4, E8>(p, num_seqs, total_q, max_q_len, stream);
    case 8: return launch_prefill_dg<D, 8, E8>(p, num_seqs, total_q, max_q_len, stream);
    case 16: return launch_prefill_dg<D, 16, E8>(p, num_seqs, total_q, max_q_len, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_varlen_prefill(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs, int total_q,
                                 int max_q_len, hipStream_t stream) {
  if (max_q_len <= 1) return hipSuccess;  // no sequence has two or more query tokens
  const bool e8 = kv_kind == KV_E5M2;
  if (!e8 && kv_kind != KV_BF16) return hipErrorInvalidValue;
  if (head_dim == 128)
    return e8 ? launch_prefill_d<128, true>(p, gqa, num_seqs, total_q, max_q_len, stream)
              : launch_prefill_d<128, false>(p, gqa, num_seqs, total_q, max_q_len, stream);
  if (head_dim == 64)
    return e8 ? launch_prefill_d<64, true>(p, gqa, num_seqs, total_q, max_q_len, stream)
              : launch_prefill_d<64, false>(p, gqa, num_seqs, total_q, max_q_len, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
