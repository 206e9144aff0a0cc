// Multi-token decode of a packed (varlen) step on gfx950 MFMA: sequences that attend a few new
// tokens at once, n * G <= 16 * NT query rows per KV head (speculative verification of draft
// tokens, short prefill chunks).
//
// Same attention as the prefill tiles (Colossal-Inference release post, "连续批量化算法
// (Continuous Batching)": packed 1-D rows; LLM inference optimisation overview, 2.2.2 "GQA"
// and 2.2.1 "Flash Attention": the G heads of a group share the K/V, softmax reduced block by
// block), but shaped like decode: with few query rows the cost is streaming each (sequence,
// KV head) context once, so one work-group takes one context and its 4 waves split the
// context's 16-key cache blocks (block b goes to wave b % 4), merging through LDS at the end.
//
// Per block and 16-row tile, with lane l, lg = l / 16:
//   S^T[16 keys][16 rows] = K . Q^T       v_mfma_f32_16x16x32_bf16 x (D / 32); A = K straight
//                                          from global memory (lane l: key l % 16, dims
//                                          32 kk + 8 lg ..), B = Q from registers
//   O^T[D][16 rows]      += V^T . P^T     v_mfma_f32_16x16x16_bf16 x (D / 16); B = P^T is the
//                                          S^T accumulator itself (lane l: keys 4 lg .. 4 lg + 3
//                                          of row l % 16, rounded to bf16), A = V^T read from
//                                          the wave's own row-major copy of the block in LDS with
//                                          ds_read_b64_tr_b16
// Row sums come from the same rounded weights through an MFMA with a ones matrix.
//
// The same body serves the decode calls when a KV head is shared by 8 or more query heads (DEC):
// one query row per sequence, whose G heads are the rows of the tile, over the decode grid
// (KV head, partition, sequence).  There the vector-ALU decode kernel spends two f32 FMAs per
// head per element; the matrix cores take the products, and only the widening and the softmax are
// left to the vector ALU.  A split partition writes its rows' (o/l, m, l) to the decode workspace
// for the reduce kernel, and the append of the newest token is done here as in the vector kernel:
// the work-group whose range holds position L-1 stores the new rows (cast to E5M2 for that cache)
// and uses the same cast values for that token instead of reading its slot back.
#include <atomic>
#include <type_traits>

#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 mq_bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float mq_f32x4_t;
typedef short mq_v4i16_t __attribute__((ext_vector_type(4)));

constexpr float kTauMq = 8.0f;
constexpr int kMaxRankedMq = 1024;
static_assert(kLongestFirstMaxSeqs <= kMaxRankedMq, "the ranking buffer holds every ranked sequence");

typedef __attribute__((ext_vector_type(8))) _Float16 mq_f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 mq_f16x4_t;

// bf16 MFMAs, or f16 ones for an E5M2 cache (E8)
template <bool E8>
__device__ __forceinline__ mq_f32x4_t mfma_k32(const uint4& a, const uint4& b, const mq_f32x4_t& c) {
  if constexpr (E8)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mq_f16x8_t, a), __builtin_bit_cast(mq_f16x8_t, b),
                                                  c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mq_bf16x8_t, a),
                                                   __builtin_bit_cast(mq_bf16x8_t, b), c, 0, 0, 0);
}
template <bool E8>
__device__ __forceinline__ mq_f32x4_t mfma_k16(const uint2& a, const uint2& b, const mq_f32x4_t& c) {
  if constexpr (E8)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(mq_f16x4_t, a), __builtin_bit_cast(mq_f16x4_t, b),
                                                 c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mq_v4i16_t, a),
                                                     __builtin_bit_cast(mq_v4i16_t, b), c, 0, 0, 0);
}
// ds_read_b64_tr_b16: within each 16-lane group, lane i's j-th 16-bit result is element i % 4 of
// the 8 bytes read by lane 4 j + i / 4 (checked on the device)
__device__ __forceinline__ uint2 mq_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) mq_v4i16_t lds_v4i16_t;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p)));
}

__device__ __forceinline__ const int32_t* table_of(const DecodeParams& p, int s) {
  return p.block_tables + (size_t)s * p.max_blocks_per_seq;
}

}  // namespace

// E8: the cache holds E5M2 codes, widened to f16 as they are loaded; queries and probabilities
// in f16 and the products on the f16 MFMA.  DEC: the decode calls (see above).
template <int D, int G, int NT, bool E8, bool DEC, int W = 4>
__device__ __forceinline__ void mq_body(const DecodeParams& p) {
  constexpr int ROWS = NT * 16;       // query rows of the work-group: row r = (token r / G, head r % G)
  constexpr int KS = D / 32;          // k-steps of the QK product
  constexpr int DT = D / 16;          // 16-dim output tiles
  constexpr int CH = D / 8;           // 16-byte chunks per cache row
  constexpr int VP = D + 16;          // row pitch of a wave's V copy (bf16): conflict-free transposed reads
  constexpr int VLD = 16 * CH / 64;   // 16-byte V chunks per lane per block
  constexpr int VWAVE = 16 * VP;      // bf16 per wave's V copy
  // one wave (split partitions only) needs neither the merge nor the longest-first ranking
  constexpr int MERGE_BYTES = W > 1 ? W * ROWS * (D + 2) * 4 : 0;  // each wave's o, m, l
  constexpr int STREAM_BYTES = W * VWAVE * 2 + (W > 1 ? 2 * kMaxRankedMq * 4 : 0);
  constexpr int LDS_BYTES = MERGE_BYTES > STREAM_BYTES ? MERGE_BYTES : STREAM_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int hq = p.num_kv_heads * G;

  int s = blockIdx.z, g = blockIdx.x;
  const int part = DEC ? blockIdx.y : 0;
  if (W > 1 && p.longest_first) {
    int* len = reinterpret_cast<int*>(lds + W * VWAVE * 2);
    const int2 u = longest_first_unit<64 * W>(p.context_lens, gridDim.z, gridDim.x, p.snake, len, len + kMaxRankedMq);
    s = u.x;
    g = u.y;
  }
  int a, n;
  if constexpr (DEC) {
    a = s;  // the sequence's one query row
    n = 1;
  } else {
    a = load_invariant(p.cu_q + s);
    n = load_invariant(p.cu_q + s + 1) - a;
    if (n <= 1) return;  // single rows: the decode kernel
  }
  int L = load_invariant(p.context_lens + s);
  L = L < 0 ? 0 : L;
  L = L > p.max_context_len ? p.max_context_len : L;
  L = L > p.max_blocks_per_seq * 16 ? p.max_blocks_per_seq * 16 : L;
  const bool causal = DEC || p.causal != 0;
  // keys [t0, t1) of this work-group: a decode partition, else the whole context
  int t0 = 0, t1 = L, nparts = 1;
  if (DEC && p.partition_tokens > 0) {
    t0 = part * p.partition_tokens;
    t1 = min(L, t0 + p.partition_tokens);
    nparts = (L + p.partition_tokens - 1) / p.partition_tokens;
    if (part > 0 && t0 >= L) return;
  }

  // ---- query rows (B operand of S^T = K Q^T) ----------------------------------------------
  int tok[NT], lim[NT];
  uint4 qb[NT][KS];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = j * 16 + lr;
    tok[j] = r / G;
    const bool ok = tok[j] < n;
    lim[j] = ok ? min(t1, causal ? min(L, L - n + tok[j] + 1) : L) : 0;  // keys [0, lim) visible
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(p.query) + ((size_t)(a + (ok ? tok[j] : 0)) * hq + (size_t)g * G + r % G) * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * kk + 8 * lg);
      if constexpr (E8)
        v = make_uint4(pack_f16x2_rne(bf16lo(v.x), bf16hi(v.x)), pack_f16x2_rne(bf16lo(v.y), bf16hi(v.y)),
                       pack_f16x2_rne(bf16lo(v.z), bf16hi(v.z)), pack_f16x2_rne(bf16lo(v.w), bf16hi(v.w)));
      qb[j][kk] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  }
  // the keys every valid row of the work-group sees: blocks below need no mask
  const int last_tok = min(n, ROWS / G) - 1;
  const int lim_min = min(t1, causal ? min(L, L - n + 1) : L);  // token 0
  const int kv_end = max(0, min(t1, causal ? min(L, L - n + last_tok + 1) : L));

  float m_run[NT];
  mq_f32x4_t lacc[NT], oacc[NT][DT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    m_run[j] = -__builtin_inff();
    lacc[j] = mq_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[j][dt] = mq_f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  constexpr uint32_t ONE2 = E8 ? 0x3C003C00u : 0x3F803F80u;  // (f16 or bf16) 1.0 x2
  const uint2 kOnes = make_uint2(ONE2, ONE2);
  constexpr int SZ = E8 ? 1 : 2;  // cache bytes per element

  const int* table = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(p.key_cache);
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(p.value_cache);
  const size_t blk_bytes = (size_t)p.num_kv_heads * 16 * D * SZ;
  const uint32_t k_off = (uint32_t)(((g * 16 + lr) * D + 8 * lg) * SZ);  // + 32 kk elements
  uint32_t v_off[VLD];
  int v_lds[VLD];
#pragma unroll
  for (int u = 0; u < VLD; ++u) {
    const int q = lane + 64 * u, key = q / CH, c = q % CH;
    v_off[u] = (uint32_t)(((g * 16 + key) * D + c * 8) * SZ);
    v_lds[u] = key * VP + c * 8;
  }
  uint16_t* vs = reinterpret_cast<uint16_t*>(lds) + wave * VWAVE;
  // lane m of group lg reads key 4 lg + m / 4, dims dt * 16 + 4 (m % 4): V^T for dims dt*16 + lr
  const int v_rd = (4 * lg + (lr >> 2)) * VP + 4 * (lr & 3);

  // ---- the newest token (DEC with key_new): its rows in this lane's K and V layouts -------
  const bool appending = DEC && p.key_new != nullptr && L - 1 >= t0 && L - 1 < t1;
  const int b_new = appending ? (L - 1) / 16 : -1;
  const int r_new = (L - 1) & 15;
  // 8 bf16 as the cache holds them (bf16, or the E5M2 cast widened to f16: a code is the upper
  // byte of the f16 of the same value)
  auto cast8 = [](uint4 v) {
    if constexpr (E8) {
      auto c = [](uint32_t w) { return (bf16_to_e5m2(w & 0xFFFFu) << 8) | (bf16_to_e5m2(w >> 16) << 24); };
      return make_uint4(c(v.x), c(v.y), c(v.z), c(v.w));
    } else {
      return v;
    }
  };
  const uint16_t* kr = reinterpret_cast<const uint16_t*>(p.key_new) + ((size_t)s * p.num_kv_heads + g) * D;
  const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.value_new) + ((size_t)s * p.num_kv_heads + g) * D;
  if (appending) {
    // the slot, written by wave 0 in the cache's format (nothing in this launch reads it back)
    const int phys = load_invariant(table_of(p, s) + b_new);
    if (wave == 0 && lane < CH && phys >= 0 && phys < p.num_blocks) {
      const size_t el = (((size_t)phys * p.num_kv_heads + g) * 16 + r_new) * D + lane * 8;
      const uint4 kv = cast8(*reinterpret_cast<const uint4*>(kr + lane * 8));
      const uint4 vv = cast8(*reinterpret_cast<const uint4*>(vr + lane * 8));
      if constexpr (E8) {
        auto pk = [](uint32_t lo, uint32_t hi) { return (lo >> 8 & 0xFFu) | (lo >> 16 & 0xFF00u) | (hi << 8 & 0xFF0000u) | (hi & 0xFF000000u); };
        *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(p.key_cache_w) + el) = make_uint2(pk(kv.x, kv.y), pk(kv.z, kv.w));
        *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(p.value_cache_w) + el) = make_uint2(pk(vv.x, vv.y), pk(vv.z, vv.w));
      } else {
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.key_cache_w) + el) = kv;
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.value_cache_w) + el) = vv;
      }
    }
  }

  struct Block {
    uint4 k[KS];
    uint4 v[VLD];
    bool ok;
  };
  auto load_block = [&](int b, Block& t) __attribute__((always_inline)) {
    int phys = load_invariant(table + b);
    t.ok = phys >= 0 && phys < p.num_blocks;
    phys = t.ok ? phys : 0;
    const uint8_t* kb = kc + (size_t)phys * blk_bytes;
    const uint8_t* vb = vc + (size_t)phys * blk_bytes;
    // 8 elements as bf16 (or f16 widened from E5M2).  STREAM: a streaming load for data read once in
    // whole lines (V: each load covers four whole rows).  A K load covers only a 64-byte half of
    // each of its 16 rows' lines, the other half coming with the next k-step's load, so K is read
    // through the cache normally: a streamed half-line could be gone before its second half is
    // asked for, and the line would be fetched twice.
    auto ld16 = [](const uint8_t* q, auto nt) {
      constexpr bool STREAM = decltype(nt)::value;
      if constexpr (E8) {
        const u32x2_t v = ld<u32x2_t, STREAM>(q);
        return make_uint4(e5m2_pair_lo(v.x), e5m2_pair_hi(v.x), e5m2_pair_lo(v.y), e5m2_pair_hi(v.y));
      } else {
        const u32x4_t v = ld<u32x4_t, STREAM>(q);
        return make_uint4(v.x, v.y, v.z, v.w);
      }
    };
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) t.k[kk] = ld16(kb + k_off + 32 * kk * SZ, std::false_type{});
#pragma unroll
    for (int u = 0; u < VLD; ++u) t.v[u] = ld16(vb + v_off[u], std::true_type{});
    __builtin_amdgcn_sched_barrier(0);  // issue the block before the math that follows
    if (b == b_new) {  // the appended token: its rows, not the slot being written
      // read here, not held in registers across the stream (a select between two arrays of
      // rows would put both in scratch)
      if (lr == r_new) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) t.k[kk] = cast8(*reinterpret_cast<const uint4*>(kr + 32 * kk + 8 * lg));
      }
#pragma unroll
      for (int u = 0; u < VLD; ++u)
        if ((lane + 64 * u) / CH == r_new) t.v[u] = cast8(*reinterpret_cast<const uint4*>(vr + ((lane + 64 * u) % CH) * 8));
    }
  };

  auto compute_block = [&](int b, Block& t) __attribute__((always_inline)) {
    // the wave's V copy.  Rows past the context must read as zeros (the pool may hold NaN there);
    // only a context's last block has such rows, so every block is copied as loaded and that one
    // then has its dead rows overwritten, each lane rewriting its own slots (its later store
    // wins).  A per-lane select on every block compiled to four divergent branches, and a select
    // under a wave-uniform branch to register copies before the stores.
    const int live = t.ok ? min(16, kv_end - 16 * b) : 0;
#pragma unroll
    for (int u = 0; u < VLD; ++u) *reinterpret_cast<uint4*>(vs + v_lds[u]) = t.v[u];
    if (live < 16) {
#pragma unroll
      for (int u = 0; u < VLD; ++u)
        if ((lane + 64 * u) / CH >= live) *reinterpret_cast<uint4*>(vs + v_lds[u]) = make_uint4(0, 0, 0, 0);
    }
    const bool whole = t.ok && 16 * b + 16 <= lim_min;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      mq_f32x4_t sa = mq_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) sa = mfma_k32<E8>(t.k[kk], qb[j][kk], sa);
      float sv[4];
      float mx = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * b + 4 * lg + i;
        sv[i] = (whole || (t.ok && key < lim[j])) ? sa[i] : -__builtin_inff();
        mx = fmaxf(mx, sv[i]);
      }
      // the row's running max moves only past the threshold; lanes' own maxima gate the reduction
      if (__any(mx * p.scale_log2 > m_run[j] + kTauMq)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mx *= p.scale_log2;
        const bool need = mx > m_run[j] + kTauMq;
        const float mn = need ? mx : m_run[j];
        const float alpha = need ? fast_exp2(m_run[j] - mn) : 1.f;
        lacc[j] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[j][dt] *= alpha;
        m_run[j] = mn;
      }
      const float mneg = m_run[j] == -__builtin_inff() ? 0.f : -m_run[j];
      typedef std::conditional_t<E8, _Float16, __bf16> pel_t;
      pel_t pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = (pel_t)fast_exp2(fmaf(sv[i], p.scale_log2, mneg));  // -inf -> 0
      const uint2 pt = make_uint2(
          (uint32_t)__builtin_bit_cast(uint16_t, pb[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, pb[1]) << 16),
          (uint32_t)__builtin_bit_cast(uint16_t, pb[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, pb[3]) << 16));
      lacc[j] = mfma_k16<E8>(kOnes, pt, lacc[j]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 va = mq_read_tr16(vs + v_rd + dt * 16);  // V^T[dims dt*16 + lr][keys 4lg..]
        oacc[j][dt] = mfma_k16<E8>(va, pt, oacc[j][dt]);
      }
    }
  };

  // ---- stream the context: block b on wave b % W, one block of prefetch -----------------
  const int b0 = t0 / 16;  // a partition starts on a block boundary
  const int nblk = (kv_end + 15) / 16 - b0;
  const int nb = wave < nblk ? (nblk - wave + W - 1) / W : 0;
  if (nb > 0) {
    Block x, y;
    int b = b0 + wave;
    load_block(b, x);
    int i = 0;
    for (; i + 2 < nb; i += 2) {
      load_block(b + W, y);
      compute_block(b, x);
      load_block(b + 2 * W, x);
      compute_block(b + W, y);
      b += 2 * W;
    }
    if (i + 1 < nb) {
      load_block(b + W, y);
      compute_block(b, x);
      compute_block(b + W, y);
    } else {
      compute_block(b, x);
    }
  }

  if constexpr (W == 1) {
    // one wave: its rows are the whole result; lane (lr, lg) holds dims dt*16 + 4 lg.. of row lr
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int r = j * 16 + lr, t = r / G;
      if (t >= n) continue;
      const float den = lacc[j][0];
      if (DEC && nparts > 1) {  // a split partition: (o/l, m, l) for the reduce kernel
        const size_t jj = ((size_t)s * hq + (size_t)g * G + r % G) * p.max_parts + part;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          float4 o;
          o.x = den > 0.f ? oacc[j][dt][0] / den : 0.f;
          o.y = den > 0.f ? oacc[j][dt][1] / den : 0.f;
          o.z = den > 0.f ? oacc[j][dt][2] / den : 0.f;
          o.w = den > 0.f ? oacc[j][dt][3] / den : 0.f;
          *reinterpret_cast<float4*>(p.ws_o + jj * D + dt * 16 + 4 * lg) = o;
        }
        if (lg == 0) {
          p.ws_m[jj] = m_run[j];
          p.ws_l[jj] = den;
        }
      } else {
        uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + ((size_t)(a + t) * hq + (size_t)g * G + r % G) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          uint32_t h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = f32_to_bf16_rne(den > 0.f ? oacc[j][dt][i] / den : 0.f);
          *reinterpret_cast<uint2*>(orow + dt * 16 + 4 * lg) = make_uint2(h[0] | h[1] << 16, h[2] | h[3] << 16);
        }
      }
    }
    return;
  }

  // ---- merge the waves: o (unnormalised), m, l per row through LDS ------------------------
  __syncthreads();  // the V copies are done with
  float* mo = reinterpret_cast<float*>(lds);          // [W][ROWS][D]
  float* mm = mo + W * ROWS * D;                       // [W][ROWS]
  float* ml = mm + W * ROWS;                           // [W][ROWS]
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = j * 16 + lr;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mo[(wave * ROWS + r) * D + dt * 16 + 4 * lg + i] = oacc[j][dt][i];
    if (lg == 0) {
      mm[wave * ROWS + r] = m_run[j];
      ml[wave * ROWS + r] = lacc[j][0];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < ROWS * D; idx += 64 * W) {
    const int r = idx / D, d = idx % D;
    const int t = r / G;
    if (t >= n) continue;
    float mx = mm[r];
#pragma unroll
    for (int w = 1; w < W; ++w) mx = fmaxf(mx, mm[w * ROWS + r]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = mm[w * ROWS + r];
      const float c = mw == -__builtin_inff() ? 0.f : fast_exp2(mw - mx);
      num = fmaf(c, mo[(w * ROWS + r) * D + d], num);
      den = fmaf(c, ml[w * ROWS + r], den);
    }
    const float o = den > 0.f ? num / den : 0.f;
    if (DEC && nparts > 1) {  // a split partition: (o/l, m, l) for the reduce kernel
      const size_t j = ((size_t)s * hq + (size_t)g * G + r % G) * p.max_parts + part;
      p.ws_o[j * D + d] = o;
      if (d == 0) {
        p.ws_m[j] = mx;
        p.ws_l[j] = den;
      }
    } else {
      reinterpret_cast<uint16_t*>(p.out)[((size_t)(a + t) * hq + (size_t)g * G + r % G) * D + d] =
          (uint16_t)f32_to_bf16_rne(o);
    }
  }
}

template <int D, int G, int NT, bool E8>
__global__ __launch_bounds__(256, 2) void varlen_multiquery_kernel(const DecodeParams p) {
  mq_body<D, G, NT, E8, false>(p);
}

// W waves per work-group: 4 on whole contexts, 1 per split partition (see launch_dec_dg)
template <int D, int G, bool E8, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(3))) void decode_mfma_kernel(const DecodeParams p) {
  mq_body<D, G, 1, E8, true, W>(p);
}

// ---------------------------------------------------------------------------------------------
namespace {

int mq_device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && (cus = cache[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <int D, int G, int NT, bool E8>
hipError_t launch_mq_dgn(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  auto kernel = varlen_multiquery_kernel<D, G, NT, E8>;
  DecodeParams q = p;
  q.longest_first = num_seqs <= kLongestFirstMaxSeqs ? 1 : 0;
  q.snake = 0;
  if (q.longest_first) {
    // longest first with the snake order when the whole grid is resident at once (as for the
    // decode kernel); otherwise the plain grid order
    static std::atomic<int> per_cu_cache{0};
    int per_cu = per_cu_cache.load(std::memory_order_relaxed);
    if (per_cu <= 0 &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) == hipSuccess)
      per_cu_cache.store(per_cu, std::memory_order_relaxed);
    const int cus = mq_device_cus();
    if (cus > 0 && per_cu > 0 && (long long)num_seqs * p.num_kv_heads <= (long long)cus * per_cu)
      q.snake = cus;
    else
      q.longest_first = 0;
  }
  hipLaunchKernelGGL(kernel, dim3(p.num_kv_heads, 1, num_seqs), dim3(256), 0, stream, q);
  return hipGetLastError();
}

// The decode grid (KV head, partition, sequence).  Whole contexts: 4 waves per work-group, longest
// first with the snake order when the grid is resident at once (as for the vector decode kernel).
// Split partitions: one wave per partition, whose rows are then the partition's result with no
// merge through LDS; measured on 8 x 32768 tokens in 512-token partitions (G = 8), 181 us against
// 188 us with 4 waves and 187 us with 2, while on whole contexts one wave per work-group is much
// slower (fewer waves stream each context).
template <int D, int G, bool E8>
hipError_t launch_dec_dg(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  DecodeParams q = p;
  q.snake = 0;
  if (p.partition_tokens > 0) {
    hipLaunchKernelGGL((decode_mfma_kernel<D, G, E8, 1>), dim3(p.num_kv_heads, p.max_parts, num_seqs), dim3(64), 0,
                       stream, q);
    return hipGetLastError();
  }
  auto kernel = decode_mfma_kernel<D, G, E8, 4>;
  if (q.longest_first) {
    static std::atomic<int> per_cu_cache{0};
    int per_cu = per_cu_cache.load(std::memory_order_relaxed);
    if (per_cu <= 0 && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) == hipSuccess)
      per_cu_cache.store(per_cu, std::memory_order_relaxed);
    const int cus = mq_device_cus();
    if (cus > 0 && per_cu > 0 && (long long)num_seqs * p.num_kv_heads <= (long long)cus * per_cu)
      q.snake = cus;
    else
      q.longest_first = 0;  // not all resident: plain grid order (see kLongestFirstMaxSeqs)
  }
  hipLaunchKernelGGL(kernel, dim3(p.num_kv_heads, 1, num_seqs), dim3(256), 0, stream, q);
  return hipGetLastError();
}

template <int D, bool E8>
hipError_t launch_dec_d(const DecodeParams& p, int gqa, int num_seqs, hipStream_t stream) {
  if (gqa == 8) return launch_dec_dg<D, 8, E8>(p, num_seqs, stream);
  if (gqa == 16) return launch_dec_dg<D, 16, E8>(p, num_seqs, stream);
  return hipErrorInvalidValue;
}

template <int D, int G, bool E8>
hipError_t launch_mq_dg(const DecodeParams& p, int num_seqs, int max_q_len, hipStream_t stream) {
  if (max_q_len * G <= 16) return launch_mq_dgn<D, G, 1, E8>(p, num_seqs, stream);
  return launch_mq_dgn<D, G, 2, E8>(p, num_seqs, stream);
}

template <int D, bool E8>
hipError_t launch_mq_d(const DecodeParams& p, int gqa, int num_seqs, int max_q_len, hipStream_t stream) {
  switch (gqa) {
    case 1: return launch_mq_dg<D, 1, E8>(p, num_seqs, max_q_len, stream);
    case 2: return launch_mq_dg<D, 2, E8>(p, num_seqs, max_q_len, stream);
    case 4: return launch_mq_dg<D, 4, E8>(p, num_seqs, max_q_len, stream);
    case 8: return launch_mq_dg<D, 8, E8>(p, num_seqs, max_q_len, stream);
    case 16: return launch_mq_dg<D, 16, E8>(p, num_seqs, max_q_len, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool multiquery_applies(int gqa, int max_q_len) { return max_q_len >= 2 && max_q_len * gqa <= 32; }

bool decode_mfma_applies(const DecodeParams& p, int kv_kind, int head_dim, int gqa) {
  return p.cu_q == nullptr && (kv_kind == KV_BF16 || kv_kind == KV_E5M2) && (gqa == 8 || gqa == 16) &&
         (head_dim == 64 || head_dim == 128);
}

hipError_t launch_decode_mfma(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs,
                              hipStream_t stream) {
  const bool e8 = kv_kind == KV_E5M2;
  if (head_dim == 128)
    return e8 ? launch_dec_d<128, true>(p, gqa, num_seqs, stream) : launch_dec_d<128, false>(p, gqa, num_seqs, stream);
  return e8 ? launch_dec_d<64, true>(p, gqa, num_seqs, stream) : launch_dec_d<64, false>(p, gqa, num_seqs, stream);
}

hipError_t launch_varlen_multiquery(const DecodeParams& p, int kv_kind, int head_dim, int gqa, int num_seqs,
                                    int max_q_len, hipStream_t stream) {
  if (!multiquery_applies(gqa, max_q_len)) return hipErrorInvalidValue;
  const bool e8 = kv_kind == KV_E5M2;
  if (!e8 && kv_kind != KV_BF16) return hipErrorInvalidValue;
  if (head_dim == 128)
    return e8 ? launch_mq_d<128, true>(p, gqa, num_seqs, max_q_len, stream)
              : launch_mq_d<128, false>(p, gqa, num_seqs, max_q_len, stream);
  if (head_dim == 64)
    return e8 ? launch_mq_d<64, true>(p, gqa, num_seqs, max_q_len, stream)
              : launch_mq_d<64, false>(p, gqa, num_seqs, max_q_len, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
