// Device code of the prefill rows of a packed step on MFMA, shared by the prefill kernel
// (varlen.hip) and the two-role packed-step kernel (packed.hip).
#pragma once

#include <climits>
#include <type_traits>

#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));

constexpr float kTauPrefill = 8.0f;
constexpr int kMaxScheduledSeqs = 1024;

// Work-group barrier for the K/V tiles in LDS only: every wave's LDS accesses complete, then
// s_barrier.  __syncthreads() also carries the memory model's work-group fences, whose wait for all
// outstanding global loads the compiler folds into the first wait inside the tile loop, so the next
// tile's prefetch would have to land before this tile's products start.  Nothing else crosses waves
// through memory here.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ds_read_b64_tr_b16 on an LDS address (see the lane mapping above)
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

// 16x16x32 MFMA on bf16 operands, or on f16 operands for an E5M2 cache (E8)
template <bool E8>
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint4& a, const uint4& b, const f32x4_t& c) {
  if constexpr (E8)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// 8 E5M2 codes -> 8 f16 (exact: a code is the upper byte of the f16 of the same value)
__device__ __forceinline__ uint4 widen_e5m2x8(uint2 w) {
  return make_uint4(e5m2_pair_lo(w.x), e5m2_pair_hi(w.x), e5m2_pair_lo(w.y), e5m2_pair_hi(w.y));
}
// 8 bf16 -> 8 f16, each rounded to nearest even (exact within f16's range)
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 w) {
  return make_uint4(pack_f16x2_rne(bf16lo(w.x), bf16hi(w.x)), pack_f16x2_rne(bf16lo(w.y), bf16hi(w.y)),
                    pack_f16x2_rne(bf16lo(w.z), bf16hi(w.z)), pack_f16x2_rne(bf16lo(w.w), bf16hi(w.w)));
}

// E8: the cache holds E5M2 codes; they are widened to f16 on their way into LDS, the queries
// are taken to f16 and the products run on the f16 MFMA (probabilities in f16).
// LDS of one 4-wave group of a prefill work-group, in 16-bit elements: two K and two V tiles of 64
// keys (double buffer).  The longest-first schedule's arrays use the same memory first.
template <int D>
struct PrefillSmem {
  static constexpr int KT = 64;
  // Row pitches (16-bit elements) of the K and V tiles: D + 16 for both.  Measured with
  // SQ_LDS_BANK_CONFLICT on the bf16 packed batch, a K pitch of D + 8 costs 1.1 conflict cycles
  // per LDS instruction and D + 16 none; the V pitch D + 16 puts a transposing read's 4 rows x 4
  // chunks on distinct banks.
  static constexpr int KP = D + 16;
  static constexpr int VP = D + 16;
  static constexpr int KBUF = KT * KP, VBUF = KT * VP;
  static constexpr int ELEMS = 2 * KBUF + 2 * VBUF;
  static constexpr int BYTES = 2 * ELEMS;
  // schedule: base, n, first row and index of every sequence with n >= 2, and a count per chunk
  // of 64 sequences
  static constexpr int SCHED_INTS = 4 * kMaxScheduledSeqs + kMaxScheduledSeqs / 64;
  static_assert(BYTES >= SCHED_INTS * 4, "schedule arrays fit in the tiles");
};

// One work-group of the prefill rows: with p.sched_seqs > 0 the work-group of 1-D index bx takes
// the unit of its longest-first rank; otherwise KV head bx, query tile from the end by, sequence bz
// of a grid grid_y tiles high.  lds: PrefillSmem<D>::ELEMS elements, 16-byte aligned.
template <int D, int G, bool E8>
__device__ __forceinline__ void prefill_body(const DecodeParams& p, int bx, int by, int bz, int grid_y,
                                             uint16_t* lds) {
  constexpr int NW = 4;                   // waves
  constexpr int NT = 2;                   // 16-row MFMA tiles per wave
  constexpr int ROWS = 4 * NT * 16;       // query rows per work-group
  constexpr int TOKW = ROWS / G;          // tokens per work-group
  constexpr int KT = PrefillSmem<D>::KT;  // keys per LDS tile (4 cache blocks)
  constexpr int KS = D / 32;              // MFMA k-steps over head_dim
  constexpr int DT = D / 16;              // 16-wide output tiles over head_dim
  constexpr int KP = PrefillSmem<D>::KP;  // K row pitch in LDS (bf16 elements)
  constexpr int VP = PrefillSmem<D>::VP;  // V row pitch in LDS
  constexpr int CH = D / 8;               // 16-byte chunks per K/V row
  constexpr int LOADS = KT * CH / 256;    // 16-byte chunks per thread per tile (K and V each)
  constexpr int KBUF = PrefillSmem<D>::KBUF, VBUF = PrefillSmem<D>::VBUF;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;  // MFMA row / column-in-tile and lane group
  const int hq = p.num_kv_heads * G;
  auto clamp_len = [&](int L) {
    L = L < 0 ? 0 : L;
    L = L > p.max_context_len ? p.max_context_len : L;
    return L > p.max_blocks_per_seq * 16 ? p.max_blocks_per_seq * 16 : L;
  };

  int g, tile, s, a, n, L;
  if (p.sched_seqs > 0) {
    // ---- longest-first schedule -------------------------------------------------------------
    // Sequences with n >= 2 query tokens, compacted in index order: base = L - n, n, first row
    // a, index.  Tile t of such a sequence has the sort key L - n + min(n, (t+1)*TOKW), strictly
    // increasing in t (ties between sequences: lower compacted index first).
    int* sm_base = reinterpret_cast<int*>(lds);
    int* sm_n = sm_base + kMaxScheduledSeqs;
    int* sm_a = sm_n + kMaxScheduledSeqs;
    int* sm_seq = sm_a + kMaxScheduledSeqs;
    int* sm_cnt = sm_seq + kMaxScheduledSeqs;  // per chunk of 64 sequences
    const int nseq = p.sched_seqs;
    const int nchunks = (nseq + 63) / 64;
    // every wave reads its chunks at once (wave w: chunks w, w + NW, ...)
    constexpr int CPW = (kMaxScheduledSeqs / 64 + NW - 1) / NW;
    int cb[CPW], cn[CPW], ca[CPW];
    uint64_t cbal[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int si = (wave + c * NW) * 64 + lane;
      int nn = 0, base = 0, aa = 0;
      if (si < nseq) {
        aa = p.cu_q[si];
        nn = p.cu_q[si + 1] - aa;
        base = clamp_len(p.context_lens[si]) - nn;
      }
      cbal[c] = __ballot(si < nseq && nn >= 2);
      cb[c] = base;
      cn[c] = nn;
      ca[c] = aa;
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      if (lane == 0 && wave + c * NW < nchunks) sm_cnt[wave + c * NW] = __builtin_popcountll(cbal[c]);
    __syncthreads();
    const int mine = lane < nchunks ? sm_cnt[lane] : 0;
    const int M = min(wave_sum_i32(mine), nseq);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int ch = wave + c * NW;
      if (ch < nchunks) {
        const int off = wave_sum_i32(lane < ch ? mine : 0);
        const int pos = off + __builtin_popcountll(cbal[c] & ((1ull << lane) - 1ull));
        if (((cbal[c] >> lane) & 1ull) && pos < kMaxScheduledSeqs) {
          sm_base[pos] = cb[c];
          sm_n[pos] = cn[c];
          sm_a[pos] = ca[c];
          sm_seq[pos] = ch * 64 + lane;
        }
      }
    }
    __syncthreads();
    const int pair = bx / p.num_kv_heads;
    g = bx % p.num_kv_heads;
    if (M == 0) return;
    // With at most 64 entries lane m keeps entry m in registers for the search.
    const int eb = lane < M ? sm_base[lane] : 0, en = lane < M ? sm_n[lane] : 0;
    auto tiles_gt = [&](int K, int base, int nn) {  // tiles of one sequence whose key exceeds K
      const int x = K - base;
      const int T = (nn + TOKW - 1) / TOKW;
      return x < 0 ? T : (x >= nn ? 0 : T - x / TOKW);
    };
    // number of tiles whose key exceeds K (wave-uniform)
    auto count_gt = [&](int K) {
      int c = 0;
      if (M <= 64) {
        c = tiles_gt(K, eb, en);
      } else {
        for (int m = lane; m < M; m += 64) c += tiles_gt(K, sm_base[m], sm_n[m]);
      }
      return wave_sum_i32(c);
    };
    int klo = INT_MAX, khi = INT_MIN;
    for (int m = lane; m < M; m += 64) {
      klo = min(klo, sm_base[m] + 1);
      khi = max(khi, sm_base[m] + sm_n[m]);
    }
    klo = wave_min_i32(klo);
    khi = wave_max_i32(khi);
    if (pair >= count_gt(klo - 1)) return;  // spare work-group
    // the key of the unit of rank `pair`: the largest K with more than `pair` keys >= K (the
    // count falls as K grows).
    if (M <= 16) {
      // 64 probes a round, one per lane, each counting over the entries (read from lane m): the
      // true probes are a prefix of the lanes, and the answer lies between the last true probe
      // and the next; a range of 2^18 keys takes three rounds.
      while (klo < khi) {
        const long long span = (long long)khi - klo + 1;
        const int c = klo + (int)((span * lane + 63) / 64);  // lane 0: klo, always true
        int cnt = 0;
        for (int m = 0; m < M; ++m)
          cnt += tiles_gt(c - 1, __builtin_amdgcn_readlane(eb, m), __builtin_amdgcn_readlane(en, m));
        const uint64_t bal = __ballot(c <= khi && cnt > pair);
        const int h = 63 - __builtin_clzll(bal | 1ull);
        const int lo = klo + (int)((span * h + 63) / 64);
        const int hi = h == 63 ? khi : klo + (int)((span * (h + 1) + 63) / 64) - 1;
        klo = lo;
        khi = hi;
      }
    } else {
      while (klo < khi) {
        const int mid = klo + (int)(((long long)khi - klo + 1) / 2);
        if (count_gt(mid - 1) > pair) klo = mid;
        else khi = mid - 1;
      }
    }
    const int rank_in_key = pair - count_gt(klo);  // among the tiles whose key equals klo
    int idx = -1, seen = 0;
    for (int m0 = 0; m0 < M; m0 += 64) {
      const int m = m0 + lane;
      bool has = false;
      if (m < M) {
        const int x = klo - sm_base[m], nn = sm_n[m];
        has = x == nn || (x >= TOKW && x < nn && x % TOKW == 0);
      }
      const uint64_t bal = __ballot(has);
      const int c = __builtin_popcountll(bal);
      if (rank_in_key < seen + c) {
        const bool me = has && __builtin_popcountll(bal & ((1ull << lane) - 1ull)) == rank_in_key - seen;
        idx = m0 + __builtin_ctzll(__ballot(me));
        break;
      }
      seen += c;
    }
    // wave-uniform from here on (every lane took the same branch of the search)
    idx = __builtin_amdgcn_readfirstlane(idx);
    if (idx < 0) return;  // not reached: every rank below the unit count has a unit
    s = __builtin_amdgcn_readfirstlane(sm_seq[idx]);
    a = __builtin_amdgcn_readfirstlane(sm_a[idx]);
    n = __builtin_amdgcn_readfirstlane(sm_n[idx]);
    L = __builtin_amdgcn_readfirstlane(sm_base[idx]) + n;
    const int x = klo - (L - n);
    tile = x == n ? (n + TOKW - 1) / TOKW - 1 : x / TOKW - 1;
    __syncthreads();  // the schedule's arrays are done with before the tiles reuse them
    if (s < 0 || s >= nseq || tile < 0) return;  // not reached: the search lands on a compacted entry
  } else {
    // natural order, the last query tiles of a chunk (the most keys) first
    g = bx;
    tile = grid_y - 1 - by;
    s = bz;
    a = load_invariant(p.cu_q + s);
    n = load_invariant(p.cu_q + s + 1) - a;
    L = clamp_len(load_invariant(p.context_lens + s));
  }

  if (n <= 1) return;  // decode rows: the decode kernel
  const int i0 = tile * TOKW;
  if (i0 >= n) return;
  const bool causal = p.causal != 0;
  // keys any row of this work-group may see
  const int last_tok = min(n, i0 + TOKW) - 1;
  int kv_end = causal ? L - n + last_tok + 1 : L;
  kv_end = kv_end < 0 ? 0 : (kv_end > L ? L : kv_end);

  // ---- query rows of this lane (B operand of S^T = K Q^T) -------------------------------
  int tok[NT], lim[NT];
  uint4 qb[NT][KS];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = wave * (NT * 16) + j * 16 + lr;
    tok[j] = i0 + r / G;
    const int h = r % G;
    const bool ok = tok[j] < n;
    lim[j] = ok ? (causal ? min(L, L - n + tok[j] + 1) : L) : 0;  // keys [0, lim) visible
    // A row past the chunk reads the chunk's first row instead: its scores are finite, and its
    // weights never reach an output (every key is masked for it where masking applies, and its
    // row is not stored).  Nothing here waits for the loads.
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(p.query) + ((size_t)(a + (ok ? tok[j] : 0)) * hq + (size_t)g * G + h) * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qb[j][kk] = *reinterpret_cast<const uint4*>(qrow + 32 * kk + 8 * lg);
  }

  float m_run[NT];
  f32x4_t lacc[NT];  // every element: the row's running sum of weights
  f32x4_t oacc[NT][DT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    m_run[j] = -__builtin_inff();
    lacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[j][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // keys every row of this wave sees (0 if the wave has rows past the chunk): tiles below
  // this bound need no mask
  const int tok_first = i0 + (wave * NT * 16) / G;
  const int tok_last = i0 + (wave * NT * 16 + NT * 16 - 1) / G;
  const int wave_lim_min = tok_last >= n ? 0 : (causal ? min(L, L - n + tok_first + 1) : L);
  constexpr uint32_t ONE2 = E8 ? 0x3C003C00u : 0x3F803F80u;  // (f16 or bf16) 1.0 x2
  const uint4 kOnes = make_uint4(ONE2, ONE2, ONE2, ONE2);

  const int* table = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  constexpr int SZ = E8 ? 1 : 2;  // cache bytes per element
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(p.key_cache);
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(p.value_cache);
  // The registers hold a chunk's 8 elements as loaded (8 bf16, or 8 E5M2 codes); the widening to
  // f16 and the masking of keys past the visible range happen when the chunk goes to LDS, so
  // nothing waits on the loads until then.
  using raw_t = std::conditional_t<E8, uint2, uint4>;
  auto widen = [](const raw_t& r) -> uint4 {
    if constexpr (E8)
      return widen_e5m2x8(r);
    else
      return r;
  };

  const int ntiles = (kv_end + KT - 1) / KT;

  // Tile kt+1 is fetched into registers while tile kt is multiplied; K and V chunks are taken
  // in row order (coalesced loads, one 16-byte LDS store each).
  raw_t kreg[LOADS], vreg[LOADS];
  uint32_t chunk_ok = 0;  // bit u: chunk u of the fetched tile is a visible, stored key
  int tile_whole = 0;     // every chunk of the fetched tile is (wave-uniform)
  // Chunk u of this thread is 16-byte piece tid % CH of key tid / CH + u * (256 / CH) of the
  // tile; those keys lie in cache block u * (256 / CH) / 16 + (tid / CH) / 16 of the tile,
  // the same block for the whole wave, at a fixed offset inside the block.
  const uint32_t lane_off = ((uint32_t)(g * 16 + (tid / CH) % 16)) * D + (uint32_t)(tid % CH) * 8;
  const int wave_blk = __builtin_amdgcn_readfirstlane((tid / CH) / 16);
  const size_t blk_stride = (size_t)p.num_kv_heads * 16 * D;
  // The 4 cache blocks of a tile: one wave-uniform (scalar) table read each, issued one tile
  // ahead of the loads that use them.
  struct TileBlocks {
    int ph[KT / 16];
  };
  auto read_table = [&](int kt) {
    TileBlocks t;
#pragma unroll
    for (int b = 0; b < KT / 16; ++b) {
      const int lb = kt * (KT / 16) + b;
      t.ph[b] = lb * 16 < kv_end ? load_invariant(table + lb) : -1;
    }
    return t;
  };
  auto fetch = [&](int kt, const TileBlocks& t) {
    int ph[KT / 16];
    bool all_valid = kt * KT + KT <= kv_end;
#pragma unroll
    for (int b = 0; b < KT / 16; ++b) {
      const int e = t.ph[b];
      const bool v = e >= 0 && e < p.num_blocks;
      all_valid = all_valid && v;
      ph[b] = v ? e : -1;
    }
    // block of chunk u: BPU * u + wave_blk (compile-time indices only, so ph stays in SGPRs)
    constexpr int BPU = (256 / CH) / 16;
    auto block_of = [&](int u) { return BPU == 1 ? ph[u] : (wave_blk ? ph[BPU * u + 1] : ph[BPU * u]); };
    // Every load reads a stored block: a block past the table's valid entries reads block 0
    // instead, and the chunk is zeroed on its way to LDS.  The block base is wave-uniform (scalar
    // arithmetic); only the fixed lane offset is per lane.
    uint32_t okm = 0;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int phys = block_of(u);
      const size_t base = (size_t)(phys >= 0 ? phys : 0) * blk_stride * SZ;
      kreg[u] = *reinterpret_cast<const raw_t*>(kc + base + (size_t)lane_off * SZ);
      vreg[u] = *reinterpret_cast<const raw_t*>(vc + base + (size_t)lane_off * SZ);
      const int kidx = kt * KT + (tid + 256 * u) / CH;
      okm |= (kidx < kv_end && phys >= 0 ? 1u : 0u) << u;
    }
    chunk_ok = okm;
    tile_whole = __builtin_amdgcn_readfirstlane(all_valid ? 1 : 0);
  };
  // Tile i is multiplied out of buffer i % 2 while tile i + 1 waits in registers;
  // after the multiply it goes to the other buffer (free since the previous barrier) and the loads
  // of tile i + 2 are issued: one barrier per tile.
  auto store = [&](int buf) {
    uint16_t* kd = lds + buf * KBUF;
    uint16_t* vd = lds + 2 * KBUF + buf * VBUF;
    if (tile_whole) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int q = tid + 256 * u;
        const int key = q / CH, c = q % CH;
        *reinterpret_cast<uint4*>(kd + key * KP + c * 8) = widen(kreg[u]);
        *reinterpret_cast<uint4*>(vd + key * VP + c * 8) = widen(vreg[u]);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int q = tid + 256 * u;
      const int key = q / CH, c = q % CH;
      const bool ok = (chunk_ok >> u) & 1u;  // unwritten slots may hold NaN: zero them
      *reinterpret_cast<uint4*>(kd + key * KP + c * 8) = ok ? widen(kreg[u]) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(vd + key * VP + c * 8) = ok ? widen(vreg[u]) : make_uint4(0, 0, 0, 0);
    }
  };
  // Pipeline: at the top of step i, tile i+1 (loaded during step i-1) goes to the idle LDS buffer
  // and the loads of tile i+2 are issued; tile i is multiplied out of the other buffer; one barrier
  // ends the step.  The loads then have a whole tile's products to land.  The table reads and K/V
  // loads of the first tiles are issued while the query rows are still in flight.
  TileBlocks tb_next{};
  if (ntiles > 0) {
    fetch(0, read_table(0));
    if (ntiles > 1) tb_next = read_table(1);
    store(0);
  }
  lds_barrier();
  if (ntiles > 1) {
    fetch(1, tb_next);
    if (ntiles > 2) tb_next = read_table(2);
  }
  // The query operands are ready before the tile loop (their loads waited for here, once, after
  // the first tiles' loads are on their way; over an E5M2 cache they are taken to f16 here).
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (E8) qb[j][kk] = bf16x8_to_f16(qb[j][kk]);
      asm volatile("" : "+v"(qb[j][kk].x), "+v"(qb[j][kk].y), "+v"(qb[j][kk].z), "+v"(qb[j][kk].w));
    }
  // Tile i + 1 from registers to its LDS buffers and the loads of tile i + 2 issued.
  auto advance = [&](int i) {
    if (i + 1 < ntiles) {
      store((i + 1) & 1);
      if (i + 2 < ntiles) {
        fetch(i + 2, tb_next);
        if (i + 3 < ntiles) tb_next = read_table(i + 3);
      }
    }
  };
  // Scores and weights of tile i (P, in the B-operand key order); MASKED = false for the tiles
  // that every row of the work-group sees whole (no key past any row's visible range), so their
  // code holds no masking at all.
  auto scores = [&](int i, auto masked_tag, uint4 (&pb)[NT][2]) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int kt = i;
    const uint16_t* Ks = lds + (i & 1) * KBUF;
    // ---- S^T = K Q^T for the tile's 4 groups of 16 keys ------------------------------------
    // k-step outermost: 4*NT independent accumulators between dependent MFMAs
    f32x4_t sacc[NT][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < NT; ++j) sacc[j][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint4 ka = *reinterpret_cast<const uint4*>(Ks + (m * 16 + lr) * KP + 32 * kk + 8 * lg);
#pragma unroll
        for (int j = 0; j < NT; ++j) sacc[j][m] = mfma_16x16x32<E8>(ka, qb[j][kk], sacc[j][m]);
      }
    }

    // ---- mask, online softmax (threshold rescale), P in the B-operand key order -----------
    // Masking is needed only where a row's visible range ends inside the tile.
    const bool whole = !MASKED || __builtin_amdgcn_readfirstlane(kt * KT + KT <= wave_lim_min ? 1 : 0) != 0;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (!whole) {  // the scores in place, so both cases share the code that follows
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = kt * KT + m * 16 + 4 * lg + e;
            sacc[j][m][e] = key < lim[j] ? sacc[j][m][e] : -__builtin_inff();
          }
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[j][m][e]);
      // The row's running max only moves when some score exceeds it by more than the
      // threshold; the lanes' own maxima decide whether the row maxima are needed at all.
      if (__any(mx * p.scale_log2 > m_run[j] + kTauPrefill)) {  // scale > 0
        asm volatile("");  // a real branch: the rescale is rare, so it is not executed speculatively
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mx *= p.scale_log2;
        const bool need = mx > m_run[j] + kTauPrefill;
        const float mn = need ? mx : m_run[j];
        const float alpha = need ? fast_exp2(m_run[j] - mn) : 1.f;
        lacc[j] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[j][dt] *= alpha;
        m_run[j] = mn;
      }
      const float mneg = m_run[j] == -__builtin_inff() ? 0.f : -m_run[j];
      uint32_t pk[4][2];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        typedef std::conditional_t<E8, _Float16, __bf16> pel_t;
        pel_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = (pel_t)fast_exp2(fmaf(sacc[j][m][e], p.scale_log2, mneg));  // -inf -> 0
        pk[m][0] = (uint32_t)__builtin_bit_cast(uint16_t, b[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, b[1]) << 16);
        pk[m][1] = (uint32_t)__builtin_bit_cast(uint16_t, b[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, b[3]) << 16);
      }
      pb[j][0] = make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]);  // keys 4lg.. , 16+4lg..
      pb[j][1] = make_uint4(pk[2][0], pk[2][1], pk[3][0], pk[3][1]);  // keys 32+4lg.., 48+4lg..
      // row sums of the same rounded weights, on the matrix core: ones . P^T
      lacc[j] = mfma_16x16x32<E8>(kOnes, pb[j][0], lacc[j]);
      lacc[j] = mfma_16x16x32<E8>(kOnes, pb[j][1], lacc[j]);
    }
  };
  // O^T += V^T P^T for the tile in V buffer vb.
  auto accumulate = [&](int vb, const uint4 (&pb)[NT][2]) {
    const uint16_t* Vs = lds + 2 * KBUF + vb * VBUF;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        // lane lr of group lg reads dims dt*16 + 4(lr%4).. of key ks*32 + 4lg + lr/4 (and +16)
        const uint16_t* vsrc = Vs + (ks * 32 + 4 * lg + (lr >> 2)) * VP + dt * 16 + 4 * (lr & 3);
        const uint2 l2 = lds_read_tr16(vsrc), h2 = lds_read_tr16(vsrc + 16 * VP);
        const uint4 va = make_uint4(l2.x, l2.y, h2.x, h2.y);  // V[keys sigma][dim dt*16 + lr]
#pragma unroll
        for (int j = 0; j < NT; ++j) oacc[j][dt] = mfma_16x16x32<E8>(va, pb[j][ks], oacc[j][dt]);
      }
    }
  };
  // tiles below the smallest visible range of the work-group's rows (its first token's) are whole
  const int wg_lim_min = causal ? min(L, L - n + i0 + 1) : L;
  const int kt_whole = __builtin_amdgcn_readfirstlane(min(ntiles, max(0, wg_lim_min) / KT));
  // step i: tile i's scores, weights and values, then the barrier
  auto step = [&](int i, auto masked_tag) {
    advance(i);
    uint4 pb[NT][2];
    scores(i, masked_tag, pb);
    accumulate(i & 1, pb);
    lds_barrier();
  };
  int i = 0;
  for (; i < kt_whole; ++i) step(i, std::false_type{});
  for (; i < ntiles; ++i) step(i, std::true_type{});

  // ---- normalise and store: lane l holds dims dt*16 + 4*lg .. +3 of row l%16 --------------
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const float lt = lacc[j][0];
    const int r = wave * (NT * 16) + j * 16 + lr;
    if (tok[j] >= n) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + ((size_t)(a + tok[j]) * hq + (size_t)g * G + r % G) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t w0 = pack_bf16x2(oacc[j][dt][0] * inv, oacc[j][dt][1] * inv);
      const uint32_t w1 = pack_bf16x2(oacc[j][dt][2] * inv, oacc[j][dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + dt * 16 + 4 * lg) = make_uint2(w0, w1);
    }
  }
}

}  // namespace pa
