// Device code of the decode partition pass (one work-group per (partition, KV head, sequence)),
// shared by the decode kernels (decode.hip) and the two-role packed-step kernel (packed.hip).
#pragma once

#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {

constexpr float TAU = 8.0f;
constexpr int kMaxRankedSeqs = 1024;  // longest-first ordering is used up to this batch size

#ifndef PA_NT_LOADS
#define PA_NT_LOADS true  // KV tiles are streamed once per step
#endif

template <int G>
__device__ __forceinline__ float bcast_head(float v, int h) {
  switch (h * (16 / G)) {
#define PA_C(n) \
  case n:       \
    return row_bcast<n>(v);
    PA_C(0) PA_C(1) PA_C(2) PA_C(3) PA_C(4) PA_C(5) PA_C(6) PA_C(7)
    PA_C(8) PA_C(9) PA_C(10) PA_C(11) PA_C(12) PA_C(13) PA_C(14) PA_C(15)
#undef PA_C
  }
  return v;
}
template <int G>
__device__ __forceinline__ uint32_t bcast_head_u32(uint32_t v, int h) {
  switch (h * (16 / G)) {
#define PA_C(n) \
  case n:       \
    return row_bcast_u32<n>(v);
    PA_C(0) PA_C(1) PA_C(2) PA_C(3) PA_C(4) PA_C(5) PA_C(6) PA_C(7)
    PA_C(8) PA_C(9) PA_C(10) PA_C(11) PA_C(12) PA_C(13) PA_C(14) PA_C(15)
#undef PA_C
  }
  return v;
}

// Longest-first unit of work-group j0 (= rank * hkv + KV head slot).  Every work-group ranks the
// sequences by context length (ties by index) and takes the (sequence, head) unit of its rank.
// In a packed batch (cu_q non-null) the sequences that are not 1-token rows rank last (their
// work-groups return at once), and the number of sequences that take part is counted, so that the
// snake order -- rank order mirrored on every second lap of `snake` work-groups, pairing long and
// short contexts on each CU -- is applied whenever their units fit the `resident` work-groups,
// whatever the batch's other rows.  Every thread of the work-group must call it (it synchronises).
template <int THREADS>
__device__ __forceinline__ int2 decode_unit_order(const int32_t* context_lens, const int32_t* cu_q, int n, int hkv,
                                                 int snake, int resident, int* len, int* order, int* active,
                                                 int j0) {
  for (int t = threadIdx.x; t < n; t += THREADS) {
    int L = load_invariant(context_lens + t);
    if (cu_q != nullptr && load_invariant(cu_q + t + 1) - load_invariant(cu_q + t) != 1) L = -1;
    len[t] = L;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += THREADS) {
    const int lt = len[t];
    int r = 0, inactive = 0;
    for (int u = 0; u < n; ++u) {
      const int lu = len[u];
      r += (lu > lt) | ((lu == lt) & (u < t));
      inactive += lu < 0;
    }
    order[r] = t;
    if (t == 0) *active = n - inactive;
  }
  __syncthreads();
  int j = j0;
  const int total = *active * hkv;
  if (snake > 0 && total <= resident && j < total) {
    const int lap = j / snake, pos = j % snake;
    const int lap_len = min(snake, total - lap * snake);
    if (lap & 1) j = lap * snake + (lap_len - 1 - pos);
  }
  return make_int2(order[j / hkv], j % hkv);
}

template <int KV, int D, int G>
struct DecodeTile {
  static constexpr int SZ = KvBytes<KV>::value;
  static constexpr int EPL = D / 16;          // elements per lane per token row
  static constexpr int NDW = EPL * SZ / 4;    // dwords per lane per token row
  static constexpr int NL = 4;                // loads per 16-token tile (4 rows each)
  static constexpr int QDW = KV == KV_F32 ? EPL : EPL / 2;  // q dwords per head per lane
  static constexpr bool F16_Q = KV == KV_E5M2 || Scaled<KV>::value;  // bf16 query widened to f16
  static constexpr int SCW = Scaled<KV>::value ? 4 : 1;              // scale dwords per lane per tile
  static constexpr int KTILE = KTileStride<KV, D>::value;      // key pool bytes per (block, KV head)
  static constexpr int VTILE = VTileStride<KV, D>::value;      // value pool bytes per (block, KV head)
};


// LDS of one decode work-group: the ranking arrays (ints) and the wave merge (floats).
template <int G, int D, int W>
struct DecodeSmem {
  static constexpr int INTS = 2 * kMaxRankedSeqs + 1;  // lengths, order, active count
  static constexpr int FLOATS = W * G * D + 2 * W * G;  // per wave: o [G][D], m [G], l [G]
  static constexpr int BYTES = 4 * (INTS + FLOATS);
};

// One work-group of the partition pass: KV head bx, partition by, sequence (or rank) bz of a grid
// of grid_x heads by grid_z sequences.  sm_i and sm_f are this work-group's LDS (DecodeSmem).
template <int KV, int D, int G, int W>
__device__ __forceinline__ void decode_body(const DecodeParams& p, int bx, int by, int bz, int grid_x, int grid_z,
                                            int* sm_i, float* sm_f) {
  using T = DecodeTile<KV, D, G>;
  constexpr int EPL = T::EPL, NDW = T::NDW, NL = T::NL, QDW = T::QDW, SZ = T::SZ, SCW = T::SCW;
  constexpr int S = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : 4;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane >> 4, col = lane & 15;
  int g = bx;
  const int part = by;
  const int hq = p.num_kv_heads * G;
  int s = bz;
  if (p.longest_first) {
    int* sm_len = sm_i;
    int* sm_order = sm_i + kMaxRankedSeqs;
    int* sm_active = sm_i + 2 * kMaxRankedSeqs;
    const int2 u = decode_unit_order<64 * W>(p.context_lens, p.cu_q, grid_z, grid_x, p.snake, p.resident, sm_len,
                                             sm_order, sm_active, bz * grid_x + bx);
    s = u.x;
    g = u.y;
  }

  int qrow = s;
  if (p.cu_q != nullptr) {  // packed varlen batch: this kernel serves the 1-token rows
    const int a = load_invariant(p.cu_q + s), b = load_invariant(p.cu_q + s + 1);
    if (b - a != 1) return;
    qrow = a;
  }
  int L = load_invariant(p.context_lens + s);
  L = L < 0 ? 0 : L;
  L = L > p.max_context_len ? p.max_context_len : L;
  L = L > p.max_blocks_per_seq * 16 ? p.max_blocks_per_seq * 16 : L;
  int t0 = 0, t1 = L, nparts = 1;
  if (p.partition_tokens > 0) {
    t0 = part * p.partition_tokens;
    t1 = min(L, t0 + p.partition_tokens);
    nparts = (L + p.partition_tokens - 1) / p.partition_tokens;
  }
  if (part > 0 && t0 >= L) return;

  // ---- the query group, in this lane's head order -------------------------------------
  // (raw loads only here; they are waited for after the first tile's loads are issued)
  uint32_t qv[G][QDW];
  uint32_t qraw[G][T::F16_Q ? QDW : 1];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const int h = head_of_slot<G>(col, k);
    const size_t qoff = ((size_t)qrow * hq + (size_t)g * G + h) * D + (size_t)col * EPL;
    if constexpr (KV == KV_F32) {
      load_dw<QDW>(qv[k], reinterpret_cast<const float*>(p.query) + qoff);
    } else if constexpr (KV == KV_BF16) {
      load_dw<QDW>(qv[k], reinterpret_cast<const uint16_t*>(p.query) + qoff);
    } else {
      load_dw<QDW>(qraw[k], reinterpret_cast<const uint16_t*>(p.query) + qoff);
    }
  }
  // ---- append mode: the newest token's K/V row ----------------------------------------
  // Only the work-group whose partition holds position L-1 appends; its row r_new of tile
  // b_new then comes from the new row instead of the cache (no read-after-write inside
  // the launch).  Lane (row, col) keeps columns col*EPL .. col*EPL+EPL-1 in cache format.
  const int pos_new = L - 1;
  const bool appending = p.key_new != nullptr && pos_new >= t0 && pos_new < t1;
  const int b_new = appending ? pos_new / 16 : -1;
  const int r_new = pos_new & 15;
  uint32_t knew[NDW], vnew[NDW];
  constexpr bool RAW = KV == KV_E5M2 || Scaled<KV>::value;  // the new row arrives as bf16 and is cast
  uint32_t kraw[RAW ? 2 * NDW : 1], vraw[RAW ? 2 * NDW : 1];
  if (appending) {
    const size_t roff = ((size_t)s * p.num_kv_heads + g) * D + (size_t)col * EPL;  // element offset
    if constexpr (KV == KV_F32) {
      load_dw<NDW>(knew, reinterpret_cast<const float*>(p.key_new) + roff);
      load_dw<NDW>(vnew, reinterpret_cast<const float*>(p.value_new) + roff);
    } else if constexpr (KV == KV_BF16) {
      load_dw<NDW>(knew, reinterpret_cast<const uint16_t*>(p.key_new) + roff);
      load_dw<NDW>(vnew, reinterpret_cast<const uint16_t*>(p.value_new) + roff);
    } else if constexpr (RAW) {  // E5M2, INT8, E4M3: bf16 rows
      load_dw<2 * NDW>(kraw, reinterpret_cast<const uint16_t*>(p.key_new) + roff);
      load_dw<2 * NDW>(vraw, reinterpret_cast<const uint16_t*>(p.value_new) + roff);
    }
  }
  // Once the first tile is in flight: cast the new row to the cache type (bf16 -> E5M2 is
  // the cache write's own cast; INT8 and E4M3 rows are quantised with the cache write's rule, the
  // row's amax reduced over the 16 lanes of a DPP row) and store it at its slot.
  float kscale = 0.f, vscale = 0.f;  // INT8, E4M3: the new rows' scales
  auto finish_append = [&]() {
    if (!appending) return;
    if constexpr (Scaled<KV>::value) {
      auto quantize_row = [&](const uint32_t(&raw)[2 * NDW], uint32_t(&codes)[NDW]) -> float {
        int key_max = -1;
#pragma unroll
        for (int j = 0; j < 2 * NDW; ++j) key_max = max(key_max, max(bf16_mag_key(raw[j]), bf16_mag_key(raw[j] >> 16)));
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) key_max = max(key_max, __shfl_xor(key_max, off));
        const float amax = q8_amax(key_max);
        const float inv = q8_inv<KV>(amax);
#pragma unroll
        for (int j = 0; j < NDW; ++j)
          codes[j] = q8_code<KV>(bf16lo(raw[2 * j]), inv) | (q8_code<KV>(bf16hi(raw[2 * j]), inv) << 8) |
                     (q8_code<KV>(bf16lo(raw[2 * j + 1]), inv) << 16) |
                     (q8_code<KV>(bf16hi(raw[2 * j + 1]), inv) << 24);
        return amax / Q8Range<KV>::value;
      };
      kscale = quantize_row(kraw, knew);
      vscale = quantize_row(vraw, vnew);
    } else if constexpr (KV == KV_E5M2) {
#pragma unroll
      for (int j = 0; j < NDW; ++j) {
        knew[j] = bf16_to_e5m2(kraw[2 * j] & 0xFFFFu) | (bf16_to_e5m2(kraw[2 * j] >> 16) << 8) |
                  (bf16_to_e5m2(kraw[2 * j + 1] & 0xFFFFu) << 16) | (bf16_to_e5m2(kraw[2 * j + 1] >> 16) << 24);
        vnew[j] = bf16_to_e5m2(vraw[2 * j] & 0xFFFFu) | (bf16_to_e5m2(vraw[2 * j] >> 16) << 8) |
                  (bf16_to_e5m2(vraw[2 * j + 1] & 0xFFFFu) << 16) | (bf16_to_e5m2(vraw[2 * j + 1] >> 16) << 24);
      }
    }
    const int phys = load_invariant(p.block_tables + (size_t)s * p.max_blocks_per_seq + b_new);
    if (wave == 0 && row == 0 && phys >= 0 && phys < p.num_blocks) {
      const size_t unit = (size_t)phys * p.num_kv_heads + g;
      const size_t ktile = unit * T::KTILE, vtile = unit * T::VTILE;
      const size_t in_tile = ((size_t)r_new * D + (size_t)col * EPL) * SZ;
      if constexpr (Scaled<KV>::value) {
        if (col == 0) {
          float* sc = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(p.key_cache_w) + ktile +
                                               q8_scale_offset<D>(r_new));
          sc[0] = kscale;
          sc[kValueScaleOffset / 4] = vscale;
        }
      }
      uint32_t* kc = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(p.key_cache_w) + ktile + in_tile);
      uint32_t* vc = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(p.value_cache_w) + vtile + in_tile);
#pragma unroll
      for (int j = 0; j < NDW; ++j) {
        kc[j] = knew[j];
        vc[j] = vnew[j];
      }
    }
  };

  // After the first tile is in flight: widen a bf16 query to f16 pairs for an E5M2 cache,
  // and make every query register ready before the tile loop (so that the loop's own
  // waits only count tile loads).
  // INT8: the keys enter the dot products as 1152 + code (see i8_biased_lo); q_bias is
  // -1152 * sum_d q[h][d] for the head h whose score this lane holds after the row reduction.
  float q_bias = 0.f;
  auto finish_query = [&]() {
    if constexpr (T::F16_Q) {
#pragma unroll
      for (int k = 0; k < G; ++k)
#pragma unroll
        for (int j = 0; j < QDW; ++j) qv[k][j] = pack_f16x2_rne(bf16lo(qraw[k][j]), bf16hi(qraw[k][j]));
    }
    if constexpr (KV == KV_I8) {
      float qs[G];
#pragma unroll
      for (int k = 0; k < G; ++k) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < QDW; ++j) a += f16lo(qv[k][j]) + f16hi(qv[k][j]);
        qs[k] = a;
      }
      row_reduce_heads<G>(qs);
      q_bias = -1152.0f * qs[0];
    }
#pragma unroll
    for (int k = 0; k < G; ++k)
#pragma unroll
      for (int j = 0; j < QDW; ++j) asm volatile("" ::"v"(qv[k][j]));
  };

  float m_own = -__builtin_inff();  // running max (log2 domain) of this row's own head
  float l_own = 0.f;                // running sum of 2^(S - m_own) over this row's tokens
  // INT8 values enter the PV products as 1152 + code: w_own is the running sum of this row's
  // f16 weights p * scale (own head), and 1152 * w_own is taken off the accumulators at the end
  float w_own = 0.f;
  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

  const int b_first = t0 / 16 + wave;
  const int b_end = (t1 + 15) / 16;
  const int* table = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.key_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.value_cache);
  const size_t lane_off = ((size_t)row * D + (size_t)col * EPL) * SZ;

  // scales of this lane's row (INT8, E4M3): tokens row, row+4, row+8, row+12 of the tile; the key
  // scales, then 64 bytes further the value scales, both in the key pool's tile
  const size_t scale_off = (size_t)16 * D + (size_t)row * 16;

  auto load_tile = [&](int b, uint32_t (&kd)[NL][NDW], uint32_t (&vd)[NL][NDW], uint32_t (&ks)[SCW],
                       uint32_t (&vs)[SCW]) -> int {
    int phys = load_invariant(table + b);
    const bool ok = phys >= 0 && phys < p.num_blocks;
    phys = ok ? phys : 0;
    const size_t unit = (size_t)phys * p.num_kv_heads + g;
    const size_t ktile = unit * T::KTILE, vtile = unit * T::VTILE;
#pragma unroll
    for (int i = 0; i < NL; ++i) load_dw<NDW, PA_NT_LOADS>(kd[i], kbase + ktile + lane_off + (size_t)i * 4 * D * SZ);
    if constexpr (Scaled<KV>::value) load_dw<4, PA_NT_LOADS>(ks, kbase + ktile + scale_off);
#pragma unroll
    for (int i = 0; i < NL; ++i) load_dw<NDW, PA_NT_LOADS>(vd[i], vbase + vtile + lane_off + (size_t)i * 4 * D * SZ);
    if constexpr (Scaled<KV>::value) load_dw<4, PA_NT_LOADS>(vs, kbase + ktile + scale_off + kValueScaleOffset);
    __builtin_amdgcn_sched_barrier(0);  // issue the tile before any math that follows
    return ok;
  };

  auto compute_tile = [&](int b, bool ok, uint32_t (&kd)[NL][NDW], uint32_t (&vd)[NL][NDW], uint32_t (&ks)[SCW],
                          uint32_t (&vs)[SCW]) {
    // valid tokens of this tile: [b*16, min(b*16+16, t1)), all of them if the block is valid
    const int tok_lim = ok ? min(16, t1 - b * 16) : 0;
    if (b == b_new) {  // the appended token: use its row, not the (not yet written) slot
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const bool mine = (4 * i + row) == r_new;
#pragma unroll
        for (int j = 0; j < NDW; ++j) {
          kd[i][j] = mine ? knew[j] : kd[i][j];
          vd[i][j] = mine ? vnew[j] : vd[i][j];
        }
        if constexpr (Scaled<KV>::value) {
          ks[i] = mine ? as_u32(kscale) : ks[i];
          vs[i] = mine ? as_u32(vscale) : vs[i];
        }
      }
    }
    float sc[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float r[G];
      uint32_t kh[Scaled<KV>::value ? 2 * NDW : 1];  // codes of this token as f16 pairs
      if constexpr (KV == KV_I8) {  // biased: 1152 + code
#pragma unroll
        for (int j = 0; j < NDW; ++j) {
          const uint32_t wx = kd[i][j] ^ 0x80808080u;
          kh[2 * j] = i8_biased_lo(wx);
          kh[2 * j + 1] = i8_biased_hi(wx);
        }
      } else if constexpr (KV == KV_E4M3) {
#pragma unroll
        for (int j = 0; j < NDW; ++j) {
          kh[2 * j] = e4m3_pair<false>(kd[i][j]);
          kh[2 * j + 1] = e4m3_pair<true>(kd[i][j]);
        }
      }
#pragma unroll
      for (int k = 0; k < G; ++k) {
        float a = 0.f;
        if constexpr (Scaled<KV>::value) {
          a = dot2_f16_first(qv[k][0], kh[0]);
#pragma unroll
          for (int j = 1; j < 2 * NDW; ++j) a = dot2_f16(qv[k][j], kh[j], a);
        } else if constexpr (KV == KV_F32) {
#pragma unroll
          for (int j = 0; j < EPL; ++j) a = fmaf(as_f32(qv[k][j]), as_f32(kd[i][j]), a);
        } else if constexpr (KV == KV_BF16) {
          a = dot2_bf16_first(qv[k][0], kd[i][0]);
#pragma unroll
          for (int j = 1; j < NDW; ++j) a = dot2_bf16(qv[k][j], kd[i][j], a);
        } else {
          a = dot2_f16_first(qv[k][0], e5m2_pair_lo(kd[i][0]));
          a = dot2_f16(qv[k][1], e5m2_pair_hi(kd[i][0]), a);
#pragma unroll
          for (int j = 1; j < NDW; ++j) {
            a = dot2_f16(qv[k][2 * j], e5m2_pair_lo(kd[i][j]), a);
            a = dot2_f16(qv[k][2 * j + 1], e5m2_pair_hi(kd[i][j]), a);
          }
        }
        r[k] = a;
      }
      row_reduce_heads<G>(r);
      const bool live = (4 * i + row) < tok_lim;
      if constexpr (KV == KV_I8) {
        sc[i] = live ? (r[0] + q_bias) * (as_f32(ks[i]) * p.scale_log2) : -__builtin_inff();
      } else if constexpr (KV == KV_E4M3) {
        sc[i] = live ? r[0] * (as_f32(ks[i]) * p.scale_log2) : -__builtin_inff();
      } else {
        sc[i] = live ? r[0] * p.scale_log2 : -__builtin_inff();
      }
    }
    // online softmax for this row's own head, threshold rescale
    float bmax = sc[0];
#pragma unroll
    for (int i = 1; i < NL; ++i) bmax = fmaxf(bmax, sc[i]);
    const bool need = bmax > m_own + TAU;
    if (__any(need)) {
      const float mn = need ? bmax : m_own;
      const float alpha = need ? fast_exp2(m_own - mn) : 1.f;
      l_own *= alpha;
      if constexpr (KV == KV_I8) w_own *= alpha;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ah = bcast_head<G>(alpha, h);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= ah;
      }
      m_own = mn;
    }
    float pr[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) pr[i] = (4 * i + row) < tok_lim ? fast_exp2(sc[i] - m_own) : 0.f;
    // tail or skipped block: unwritten slots may hold anything (NaN); INT8 codes are always
    // finite, and there the scale is masked instead (below); E4M3 codes can be NaN
    if (KV != KV_I8 && tok_lim < 16) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const bool live = (4 * i + row) < tok_lim;
#pragma unroll
        for (int j = 0; j < NDW; ++j) vd[i][j] = live ? vd[i][j] : 0u;
      }
    }
    if constexpr (KV == KV_I8) {
#pragma unroll
      for (int i = 0; i < NL; i += 2) {
        const float w0 = (4 * i + row) < tok_lim ? pr[i] * as_f32(vs[i]) : 0.f;
        const float w1 = (4 * i + 4 + row) < tok_lim ? pr[i + 1] * as_f32(vs[i + 1]) : 0.f;
        l_own += pr[i] + pr[i + 1];
        const uint32_t pp = pack_f16x2_rne(w0, w1);
        w_own = dot2_f16(pp, 0x3C003C00u, w_own);  // + both f16 weights (times 1.0)
        uint32_t vp[EPL];
#pragma unroll
        for (int j = 0; j < NDW; ++j) {
          vp[4 * j + 0] = i8_biased_cross_pair<0>(vd[i][j], vd[i + 1][j]);
          vp[4 * j + 1] = i8_biased_cross_pair<1>(vd[i][j], vd[i + 1][j]);
          vp[4 * j + 2] = i8_biased_cross_pair<2>(vd[i][j], vd[i + 1][j]);
          vp[4 * j + 3] = i8_biased_cross_pair<3>(vd[i][j], vd[i + 1][j]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint32_t ph = bcast_head_u32<G>(pp, h);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = dot2_f16(ph, vp[e], acc[h][e]);
        }
      }
    } else if constexpr (KV == KV_E4M3) {
#pragma unroll
      for (int i = 0; i < NL; i += 2) {
        const float w0 = (4 * i + row) < tok_lim ? pr[i] * as_f32(vs[i]) : 0.f;
        const float w1 = (4 * i + 4 + row) < tok_lim ? pr[i + 1] * as_f32(vs[i + 1]) : 0.f;
        l_own += pr[i] + pr[i + 1];
        const uint32_t pp = pack_f16x2_rne(w0, w1);
        uint32_t vp[EPL];
#pragma unroll
        for (int j = 0; j < NDW; ++j) {
          vp[4 * j + 0] = e4m3_cross_pair<0>(vd[i][j], vd[i + 1][j]);
          vp[4 * j + 1] = e4m3_cross_pair<1>(vd[i][j], vd[i + 1][j]);
          vp[4 * j + 2] = e4m3_cross_pair<2>(vd[i][j], vd[i + 1][j]);
          vp[4 * j + 3] = e4m3_cross_pair<3>(vd[i][j], vd[i + 1][j]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint32_t ph = bcast_head_u32<G>(pp, h);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = dot2_f16(ph, vp[e], acc[h][e]);
        }
      }
    } else if constexpr (KV == KV_E5M2) {
#pragma unroll
      for (int i = 0; i < NL; i += 2) {
        const uint32_t pp = pack_f16x2_rne(pr[i], pr[i + 1]);
        l_own += f16lo(pp) + f16hi(pp);
        uint32_t vp[EPL];
#pragma unroll
        for (int j = 0; j < NDW; ++j) {
          vp[4 * j + 0] = e5m2_cross_pair<0>(vd[i][j], vd[i + 1][j]);
          vp[4 * j + 1] = e5m2_cross_pair<1>(vd[i][j], vd[i + 1][j]);
          vp[4 * j + 2] = e5m2_cross_pair<2>(vd[i][j], vd[i + 1][j]);
          vp[4 * j + 3] = e5m2_cross_pair<3>(vd[i][j], vd[i + 1][j]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint32_t ph = bcast_head_u32<G>(pp, h);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = dot2_f16(ph, vp[e], acc[h][e]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        l_own += pr[i];
        float vf[EPL];
        if constexpr (KV == KV_F32) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) vf[e] = as_f32(vd[i][e]);
        } else {
#pragma unroll
          for (int j = 0; j < NDW; ++j) {
            vf[2 * j] = bf16lo(vd[i][j]);
            vf[2 * j + 1] = bf16hi(vd[i][j]);
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ph = bcast_head<G>(pr[i], h);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
        }
      }
    }
  };

  // ---- stream the partition's tiles, one tile of prefetch per wave ----------------------
  // The steady-state loop issues the next tile's loads unconditionally, so the compiler's
  // wait counters see a fixed number of loads in flight and wait only for the tile being
  // consumed; the last one or two tiles are peeled off.
  {
    const int ntiles = b_first < b_end ? (b_end - b_first + W - 1) / W : 0;
    if (ntiles > 0) {
      uint32_t ka[NL][NDW], va[NL][NDW], kb[NL][NDW], vb[NL][NDW];
      uint32_t ksa[SCW], vsa[SCW], ksb[SCW], vsb[SCW];
      int b = b_first;
      int oka = load_tile(b, ka, va, ksa, vsa), okb;
      finish_query();
      finish_append();
      int i = 0;
      for (; i + 2 < ntiles; i += 2) {
        okb = load_tile(b + W, kb, vb, ksb, vsb);
        compute_tile(b, oka, ka, va, ksa, vsa);
        oka = load_tile(b + 2 * W, ka, va, ksa, vsa);
        compute_tile(b + W, okb, kb, vb, ksb, vsb);
        b += 2 * W;
      }
      if (i + 1 < ntiles) {
        okb = load_tile(b + W, kb, vb, ksb, vsb);
        compute_tile(b, oka, ka, va, ksa, vsa);
        compute_tile(b + W, okb, kb, vb, ksb, vsb);
      } else {
        compute_tile(b, oka, ka, va, ksa, vsa);
      }
    }
  }

  if constexpr (KV == KV_I8) {  // remove the bias the INT8 values carried into the accumulators
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float bh = -1152.0f * bcast_head<G>(w_own, h);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += bh;
    }
  }

  // ---- merge the four rows of the wave ----------------------------------------------------
  float mw = fmaxf(m_own, __shfl_xor(m_own, 16));
  mw = fmaxf(mw, __shfl_xor(mw, 32));
  const float ar = (m_own == -__builtin_inff()) ? 0.f : fast_exp2(m_own - mw);
  float lw = l_own * ar;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float ah = bcast_head<G>(ar, h);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[h][e] * ah;
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[h][e] = v;
    }
  }

  const bool final_out = nparts <= 1;
  const size_t out_row = ((size_t)qrow * hq + (size_t)g * G) * D;  // first head of the group
  const size_t ws_row = ((size_t)s * hq + (size_t)g * G) * p.max_parts;

  auto emit = [&](int h, int d, float num, float den, float mval) {
    const float o = den > 0.f ? num / den : 0.f;
    if (final_out) {
      if constexpr (KV == KV_F32) {
        reinterpret_cast<float*>(p.out)[out_row + (size_t)h * D + d] = o;
      } else {
        reinterpret_cast<uint16_t*>(p.out)[out_row + (size_t)h * D + d] = (uint16_t)f32_to_bf16_rne(o);
      }
    } else {
      const size_t j = ws_row + (size_t)h * p.max_parts + part;
      p.ws_o[j * D + d] = o;
      if (d == 0) {
        p.ws_m[j] = mval;
        p.ws_l[j] = den;
      }
    }
  };

  if constexpr (W == 1) {
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float lh = bcast_head<G>(lw, h);
        const float mh = bcast_head<G>(mw, h);
#pragma unroll
        for (int e = 0; e < EPL; ++e) emit(h, col * EPL + e, acc[h][e], lh, mh);
      }
    }
  } else {
    float(*sm_acc)[G][D] = reinterpret_cast<float(*)[G][D]>(sm_f);
    float(*sm_m)[G] = reinterpret_cast<float(*)[G]>(sm_f + W * G * D);
    float(*sm_l)[G] = reinterpret_cast<float(*)[G]>(sm_f + W * G * D + W * G);
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) sm_acc[wave][h][col * EPL + e] = acc[h][e];
      if ((col & (16 / G - 1)) == 0) {
        sm_m[wave][col / (16 / G)] = mw;
        sm_l[wave][col / (16 / G)] = lw;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
      const int h = idx / D, d = idx % D;
      float mx = sm_m[0][h];
#pragma unroll
      for (int w = 1; w < W; ++w) mx = fmaxf(mx, sm_m[w][h]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mwv = sm_m[w][h];
        const float a = (mwv == -__builtin_inff()) ? 0.f : fast_exp2(mwv - mx);
        num = fmaf(a, sm_acc[w][h][d], num);
        den = fmaf(a, sm_l[w][h], den);
      }
      emit(h, d, num, den, mx);
    }
  }

}

}  // namespace pa
