// Split-KV reduce for gfx950: the partitions of every split (sequence, query head) merged into
// its output row.
//
// What is computed (LLM inference optimisation overview, 2.2.1 "Flash Attention": softmax can
// be reduced without the whole input; each partition leaves its normalised o_j, its max m_j (in
// log2 units) and its sum l_j):
//   out = sum_j 2^(m_j - M) l_j o_j / sum_j 2^(m_j - M) l_j,  M = max_j m_j
#include <hip/hip_runtime.h>

#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {

// Merge the partitions of every (sequence, query head) that was split: M = max_j m_j,
// w_j = 2^(m_j - M) l_j, out = sum_j w_j o_j / sum_j w_j.  256 threads: NG groups of D/4
// lanes take every NG-th partition, each lane 4 dims (one 16-byte load per partition row), with
// the loop unrolled so that several partitions' loads are in flight; the groups then combine
// through LDS.  On 8 x 32768 tokens in 512-token partitions this one-pass form made the step
// 2.2 us faster than first reading every m_j for M and then the partials (184.2 against 186.4 us).
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const DecodeParams p) {
  constexpr int LPR = D / 4;     // lanes per partition row
  constexpr int NG = 256 / LPR;  // partition groups
  const int h = blockIdx.x, s = blockIdx.y;
  const int hq = gridDim.x;
  const int sub = threadIdx.x % LPR, grp = threadIdx.x / LPR;
  int qrow = s;
  if (p.cu_q != nullptr) {
    const int a = load_invariant(p.cu_q + s), b = load_invariant(p.cu_q + s + 1);
    if (b - a != 1) return;
    qrow = a;
  }
  int L = load_invariant(p.context_lens + s);
  L = L < 0 ? 0 : L;
  L = L > p.max_context_len ? p.max_context_len : L;
  L = L > p.max_blocks_per_seq * 16 ? p.max_blocks_per_seq * 16 : L;
  const int nparts = (L + p.partition_tokens - 1) / p.partition_tokens;
  if (nparts <= 1) return;
  const size_t base = ((size_t)s * hq + h) * p.max_parts;
  // One pass: each group merges its partitions online, rescaling by 2^(old max - new max) when a
  // partition raises its max, so every partition's loads issue without waiting for the global
  // max; the groups' (max, sum, numerator) then meet in LDS.
  __shared__ float sm_m[NG];
  __shared__ float sm_den[NG];
  __shared__ float4 sm_num[NG][LPR];
  const float4* wo = reinterpret_cast<const float4*>(p.ws_o);
  float gm = -__builtin_inff(), den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int j = grp; j < nparts; j += NG) {
    const float mj = p.ws_m[base + j];
    const float lj = p.ws_l[base + j];
    const float4 o = wo[(base + j) * LPR + sub];
    if (mj > gm) {  // an empty partition (m = -inf) never raises it
      const float c = fast_exp2(gm - mj);  // 0 while gm is still -inf
      den *= c;
      num.x *= c;
      num.y *= c;
      num.z *= c;
      num.w *= c;
      gm = mj;
    }
    const float w = mj == -__builtin_inff() ? 0.f : fast_exp2(mj - gm) * lj;
    den += w;
    num.x = fmaf(w, o.x, num.x);
    num.y = fmaf(w, o.y, num.y);
    num.z = fmaf(w, o.z, num.z);
    num.w = fmaf(w, o.w, num.w);
  }
  sm_num[grp][sub] = num;
  if (sub == 0) {
    sm_m[grp] = gm;
    sm_den[grp] = den;
  }
  __syncthreads();
  if (threadIdx.x >= LPR) return;
  float mx = sm_m[0];
#pragma unroll
  for (int g = 1; g < NG; ++g) mx = fmaxf(mx, sm_m[g]);
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
  float dsum = 0.f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float c = sm_m[g] == -__builtin_inff() ? 0.f : fast_exp2(sm_m[g] - mx);
    const float4 v = sm_num[g][sub];
    t.x = fmaf(c, v.x, t.x);
    t.y = fmaf(c, v.y, t.y);
    t.z = fmaf(c, v.z, t.z);
    t.w = fmaf(c, v.w, t.w);
    dsum = fmaf(c, sm_den[g], dsum);
  }
  const float o4[4] = {dsum > 0.f ? t.x / dsum : 0.f, dsum > 0.f ? t.y / dsum : 0.f, dsum > 0.f ? t.z / dsum : 0.f,
                       dsum > 0.f ? t.w / dsum : 0.f};
  const size_t orow = ((size_t)qrow * hq + h) * D + (size_t)sub * 4;
  if constexpr (OUT_BF16) {
    uint2 w2;
    w2.x = f32_to_bf16_rne(o4[0]) | (f32_to_bf16_rne(o4[1]) << 16);
    w2.y = f32_to_bf16_rne(o4[2]) | (f32_to_bf16_rne(o4[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + orow) = w2;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + orow) = make_float4(o4[0], o4[1], o4[2], o4[3]);
  }
}

hipError_t launch_decode_reduce(const DecodeParams& p, bool out_bf16, int head_dim, int num_q_heads, int num_seqs,
                                hipStream_t stream) {
  if (p.max_parts <= 1) return hipSuccess;
  dim3 grid(num_q_heads, num_seqs);
  if (head_dim == 128) {
    if (out_bf16) hipLaunchKernelGGL((decode_reduce_kernel<128, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((decode_reduce_kernel<128, false>), grid, dim3(256), 0, stream, p);
  } else if (head_dim == 64) {
    if (out_bf16) hipLaunchKernelGGL((decode_reduce_kernel<64, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((decode_reduce_kernel<64, false>), grid, dim3(256), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
