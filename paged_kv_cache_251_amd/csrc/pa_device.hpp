// Device helpers shared by the libpagedattn kernels (gfx950, wave64).
#pragma once

#include <climits>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_launch.hpp"

namespace pa {

template <int KV>
struct KvBytes;
template <>
struct KvBytes<KV_F32> { static constexpr int value = 4; };
template <>
struct KvBytes<KV_BF16> { static constexpr int value = 2; };
template <>
struct KvBytes<KV_E5M2> { static constexpr int value = 1; };
template <>
struct KvBytes<KV_I8> { static constexpr int value = 1; };
template <>
struct KvBytes<KV_E4M3> { static constexpr int value = 1; };

// Pools whose tiles carry one float32 scale per token after the codes.
template <int KV>
struct Scaled { static constexpr bool value = KV == KV_I8 || KV == KV_E4M3; };

// Bytes from the start of one (block, KV head) tile of 16 x D elements to the next.  Key pool:
// the codes, and for the scaled kinds the 16 float32 key scales and then the 16 float32 value
// scales of the same tokens (128 bytes, so every tile is a whole number of 128-byte lines and a
// work-group reading a tile never fetches a line that another tile shares).  Value pool: the
// codes only.
template <int KV, int D>
struct KTileStride {
  static constexpr int value = 16 * D * KvBytes<KV>::value + (Scaled<KV>::value ? 128 : 0);
};
template <int KV, int D>
struct VTileStride {
  static constexpr int value = 16 * D * KvBytes<KV>::value;
};

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

__device__ __forceinline__ uint32_t as_u32(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// ---------------------------------------------------------------------------
// DPP lane exchange inside one 16-lane row.  Pairings used by the reductions:
//   bit 3: row_mirror       lane i <- 15 - i
//   bit 2: row_half_mirror  lane i <- (i & 8) | (7 - (i & 7))
//   bit 1: quad_perm 2301   lane i <- i ^ 2
//   bit 0: quad_perm 1032   lane i <- i ^ 1
// Each flips the named bit of the lane index (and possibly lower bits only).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u32(v), CTRL, 0xF, 0xF, true));
}
// Every control these two take (row_mirror, row_half_mirror, quad_perm, row_newbcast) gives each
// lane a source in its own row, and all rows and banks are enabled, so no lane keeps `old`:
// bound_ctrl lets the compiler leave it unset instead of zeroing a register first.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_ROW_BCAST0 = 0x150;  // row_newbcast:n = 0x150 + n (lane n of each row)

template <int BIT>
struct PairCtrl;
template <>
struct PairCtrl<3> { static constexpr int value = DPP_ROW_MIRROR; };
template <>
struct PairCtrl<2> { static constexpr int value = DPP_ROW_HALF_MIRROR; };
template <>
struct PairCtrl<1> { static constexpr int value = DPP_QUAD_XOR2; };
template <>
struct PairCtrl<0> { static constexpr int value = DPP_QUAD_XOR1; };

// Host-visible twin of the pairings above, on a lane index within a row.
__host__ __device__ constexpr int pair_lane(int bit, int x) {
  return bit == 3 ? 15 - x : bit == 2 ? ((x & 8) | (7 - (x & 7))) : bit == 1 ? (x ^ 2) : (x ^ 1);
}

// Head held in register slot k of lane `col` (0..15) before the head-distributing
// reduction over G heads (see row_reduce_heads).
template <int G>
__device__ __forceinline__ int head_of_slot(int col, int k) {
  constexpr int S = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : 4;
  int y = col;
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (k & (G >> (s + 1))) y = pair_lane(3 - s, y);
  return S == 0 ? 0 : (y >> (4 - S));
}

// Sum G per-lane partial dot products over the 16 lanes of a row while spreading
// the heads over the lanes: on entry slot k of lane col holds the partial of head
// head_of_slot<G>(col, k); on exit r[0] holds the full sum for head col >> (4 - S)
// (S = log2 G), identical on the 16/G lanes that share that head.  Each step keeps
// the first half of the live slots and adds the partner lane's second half, so the
// row costs log2(16) steps with G-1 + (4-S) DPP adds instead of 4G.
template <int G>
__device__ __forceinline__ void row_reduce_heads(float (&r)[G]) {
  int n = G;
#define PA_STEP(BIT)                                                             \
  {                                                                              \
    if (n > 1) {                                                                 \
      const int half = n >> 1;                                                   \
      _Pragma("unroll") for (int k = 0; k < G / 2; ++k) if (k < half) r[k] +=    \
          dpp_f32<PairCtrl<BIT>::value>(r[half + k]);                            \
      n = half;                                                                  \
    } else {                                                                     \
      r[0] += dpp_f32<PairCtrl<BIT>::value>(r[0]);                               \
    }                                                                            \
  }
  PA_STEP(3) PA_STEP(2) PA_STEP(1) PA_STEP(0)
#undef PA_STEP
}

// Lane index (within a row) that holds head h's reduced value.
template <int G>
__device__ __forceinline__ constexpr int head_lane(int h) {
  return h * (16 / G);
}

// Reduction of an int over the 64 lanes of a wave, every lane receiving the result: an inclusive
// scan over each 16-lane row by row_shr 1, 2, 4, 8, the row totals carried forward by row_bcast:15
// and row_bcast:31 (rows 1, 3 and rows 2, 3), so that lane 63 ends with the whole wave's result.
// Lanes whose DPP source lies outside the row, and rows the mask leaves out, combine the identity.
template <typename Op>
__device__ __forceinline__ int wave_reduce_i32(int x, int identity, Op op) {
  x = op(x, __builtin_amdgcn_update_dpp(identity, x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(identity, x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(identity, x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(identity, x, 0x118, 0xF, 0xF, false));  // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(identity, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp(identity, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ int wave_sum_i32(int x) {
  return wave_reduce_i32(x, 0, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ int wave_min_i32(int x) {
  return wave_reduce_i32(x, INT_MAX, [](int a, int b) { return a < b ? a : b; });
}
__device__ __forceinline__ int wave_max_i32(int x) {
  return wave_reduce_i32(x, INT_MIN, [](int a, int b) { return a > b ? a : b; });
}

// Broadcast lane LANE of each 16-lane row to the whole row.
template <int LANE>
__device__ __forceinline__ float row_bcast(float v) {
  return dpp_f32<DPP_ROW_BCAST0 + LANE>(v);
}
template <int LANE>
__device__ __forceinline__ uint32_t row_bcast_u32(uint32_t v) {
  return dpp_u32<DPP_ROW_BCAST0 + LANE>(v);
}

// ---------------------------------------------------------------------------
// element conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return as_f32(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return as_f32(w & 0xFFFF0000u); }

// binary32 -> bfloat16, round to nearest even; NaN -> quiet NaN with sign.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = as_u32(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? (((u >> 16) & 0x8000u) | 0x7FC0u) : r;
}

// Two binary32 -> two bfloat16 (low, high half), round to nearest even, by the hardware
// conversion (v_cvt_pk_bf16_f32): finite values round as f32_to_bf16_rne does.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// bfloat16 (16-bit pattern) -> E5M2 code, round to nearest even, no saturation:
// a magnitude that rounds past 57344 becomes inf; NaN -> sign | 0x7F.
__device__ __forceinline__ uint32_t bf16_to_e5m2(uint32_t b) {
  const uint32_t sign = (b >> 8) & 0x80u;
  const uint32_t a = b & 0x7FFFu;
  // |x| >= 2^-14: move the exponent from bias 127 to bias 15, drop 5 mantissa bits
  const uint32_t x = a - (112u << 7);
  uint32_t qn = x >> 5;
  const uint32_t rn = x & 31u;
  qn += (rn > 16u) | ((rn == 16u) & (qn & 1u));
  qn = qn > 0x7Cu ? 0x7Cu : qn;
  // |x| < 2^-14: code = value / 2^-16 rounded to nearest even (0..4)
  const uint32_t e = a >> 7;
  const uint32_t mant = (a & 0x7Fu) | 0x80u;
  const uint32_t sh = 118u - e;  // >= 6 here
  const uint32_t shc = sh > 9u ? 9u : sh;
  uint32_t qs = mant >> shc;
  const uint32_t rs = mant & ((1u << shc) - 1u);
  const uint32_t half = 1u << (shc - 1u);
  qs += (rs > half) | ((rs == half) & (qs & 1u));
  qs = (sh > 9u || e == 0u) ? 0u : qs;
  uint32_t code = a >= (113u << 7) ? qn : qs;
  code = a > 0x7F80u ? 0x7Fu : code;
  return sign | code;
}

// Four E5M2 codes (bytes of w) -> two f16x2 words; exact (an E5M2 code is the upper
// byte of the f16 with the same value).
__device__ __forceinline__ uint32_t e5m2_pair_lo(uint32_t w) {
  return __builtin_amdgcn_perm(0u, w, 0x010C000Cu);
}
__device__ __forceinline__ uint32_t e5m2_pair_hi(uint32_t w) {
  return __builtin_amdgcn_perm(0u, w, 0x030C020Cu);
}

// (byte j of a, byte j of b) as an f16x2 word, low half from a.
template <int J>
__device__ __forceinline__ uint32_t e5m2_cross_pair(uint32_t a, uint32_t b) {
  // v_perm: bytes 0-3 select from the second source (a), 4-7 from the first (b)
  constexpr uint32_t sel = 0x0Cu | ((uint32_t)J << 8) | (0x0Cu << 16) | ((uint32_t)(4 + J) << 24);
  return __builtin_amdgcn_perm(b, a, sel);
}

// int8 codes -> f16, biased: with the sign bit of a byte flipped and 0x64 as the upper byte, an
// f16 holds 1024 + 128 + code exactly (1152 + code).
// Bytes 0, 1 (lo) or 2, 3 (hi) of a word as biased f16: with wx = w ^ 0x80808080 (each code's
// sign bit flipped) the upper byte 0x64 comes from the constant operand; a dot product against
// q then carries 1152 * sum(q), which the caller subtracts once.
__device__ __forceinline__ uint32_t i8_biased_lo(uint32_t wx) { return __builtin_amdgcn_perm(0x64646464u, wx, 0x04010400u); }
__device__ __forceinline__ uint32_t i8_biased_hi(uint32_t wx) { return __builtin_amdgcn_perm(0x64646464u, wx, 0x04030402u); }

// (byte j of a, byte j of b) as biased f16 values (1152 + code), low half from a
template <int J>
__device__ __forceinline__ uint32_t i8_biased_cross_pair(uint32_t a, uint32_t b) {
  constexpr uint32_t sel = (uint32_t)J | (0x0Cu << 8) | ((uint32_t)(4 + J) << 16) | (0x0Cu << 24);
  return __builtin_amdgcn_perm(b, a, sel) ^ 0x64806480u;
}

// FP8 E4M3 (OCP) codes -> f16x2, exact (every E4M3 value is an f16 value), by the matrix-core
// conversion unit: bytes 0, 1 (HI = false) or 2, 3 (HI = true) of w, low half from the lower byte.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}
// (byte j of a, byte j of b) as an f16x2 word, low half from a
template <int J>
__device__ __forceinline__ uint32_t e4m3_cross_pair(uint32_t a, uint32_t b) {
  constexpr uint32_t sel = (uint32_t)J | ((uint32_t)(4 + J) << 8) | (0x0Cu << 16) | (0x0Cu << 24);
  return e4m3_pair<false>(__builtin_amdgcn_perm(b, a, sel));
}

// binary32 -> E4M3 code, round to nearest even, saturating at 448; NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float y) {
  const uint32_t u = as_u32(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |y| >= 448
  if (a < 0x3C800000u)                        // |y| < 2^-6: steps of 2^-9 (8 steps = 2^-6)
    return sign | (uint32_t)rintf(as_f32(a) * 512.0f);
  const uint32_t x = a - (120u << 23);  // exponent bias 127 -> 7
  uint32_t q = x >> 20;
  const uint32_t r = x & 0xFFFFFu;
  q += (r > 0x80000u) | ((r == 0x80000u) & (q & 1u));
  return sign | (q > 0x7Eu ? 0x7Eu : q);
}

// Scaled 8-bit rows (INT8, E4M3): one float32 scale per (token, KV head) row, scale = amax / RANGE
// and code = Q(x * RANGE / amax), where amax is the largest magnitude of the row's bf16 elements
// with NaN ignored.  Both the cache write and the fused append use these, so their bytes agree.
template <int KV>
struct Q8Range {
  static constexpr float value = KV == KV_I8 ? 127.0f : 448.0f;  // largest code magnitude
};
// Order key of one bf16 element's magnitude: its 15-bit pattern, or -1 for NaN; the row's
// largest key gives amax (all NaN: key -1, amax NaN).
__device__ __forceinline__ int bf16_mag_key(uint32_t bits16) {
  const int a = (int)(bits16 & 0x7FFFu);
  return a > 0x7F80 ? -1 : a;
}
__device__ __forceinline__ float q8_amax(int key_max) {
  return key_max < 0 ? __builtin_nanf("") : as_f32((uint32_t)key_max << 16);
}
template <int KV>
__device__ __forceinline__ float q8_inv(float amax) {
  return amax > 0.f ? Q8Range<KV>::value / amax : 0.f;
}
// code byte of one element (INT8: nearest even, clamped to [-127, 127], NaN -> -127; E4M3: the
// saturating nearest-even encoder)
template <int KV>
__device__ __forceinline__ uint32_t q8_code(float x, float inv) {
  if constexpr (KV == KV_I8) {
    const float q = rintf(x * inv);
    return (uint32_t)(q != q ? -127 : (int)fminf(fmaxf(q, -127.f), 127.f)) & 0xFFu;
  } else {
    return f32_to_e4m3_sat(x * inv);
  }
}
// byte offset, inside a scaled key tile of head_dim D, of the key scale of token r of the block
// (its value scale sits 64 bytes further): token r's scale sits at index 4(r mod 4) + r/4, so a
// lane of DPP row q reads the scales of its tokens q, q+4, q+8, q+12 with one 16-byte load
template <int D>
__device__ __forceinline__ int q8_scale_offset(int r) {
  return 16 * D + 4 * (4 * (r & 3) + (r >> 2));
}
constexpr int kValueScaleOffset = 64;  // value scales after the key scales, in the key tile

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}
// The same products with no accumulator (the first step of a chain).  From a zero start the
// compiler picks the accumulating encoding and first zeroes its destination with a move; the
// three-operand form takes the 0 as an inline constant, one instruction instead of two.
__device__ __forceinline__ float dot2_bf16_first(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float dot2_f16_first(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Two binary32 -> f16x2, each rounded to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2_rne(float lo, float hi) {
  _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ float f16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// ---------------------------------------------------------------------------
// vector loads of N dwords (N = 1, 2, 4, 8); NT marks streaming data that is read once
// (the KV tiles), so it does not displace reusable lines in L2 / Infinity Cache.
// ---------------------------------------------------------------------------
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename V, bool NT>
__device__ __forceinline__ V ld(const void* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else
    return *reinterpret_cast<const V*>(p);
}

template <int N, bool NT = false>
__device__ __forceinline__ void load_dw(uint32_t (&d)[N], const void* p) {
  if constexpr (N == 1) {
    d[0] = ld<uint32_t, NT>(p);
  } else if constexpr (N == 2) {
    u32x2_t v = ld<u32x2_t, NT>(p);
    d[0] = v.x; d[1] = v.y;
  } else if constexpr (N == 4) {
    u32x4_t v = ld<u32x4_t, NT>(p);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  } else {
    u32x4_t v = ld<u32x4_t, NT>(p);
    u32x4_t w = ld<u32x4_t, NT>(reinterpret_cast<const uint8_t*>(p) + 16);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    d[4] = w.x; d[5] = w.y; d[6] = w.z; d[7] = w.w;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Read a value that no kernel of this launch writes (block tables, lengths) through the
// constant address space, so that a wave-uniform address becomes a scalar load.
template <typename T>
__device__ __forceinline__ T load_invariant(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<const __attribute__((address_space(4))) char*>(reinterpret_cast<uintptr_t>(p)));
}

// Longest-first work order over (sequence, KV head) units.  Ranks the n sequences by context
// length (rank of t = #{t' : L[t'] > L[t] or (L[t'] == L[t] and t' < t)}) in LDS (`len`,
// `order`: n ints each, n <= their size) and returns the unit of work-group
// j = blockIdx.z * hkv + blockIdx.x: sequence of rank j / hkv, KV head j % hkv.  With snake > 0
// (every work-group of the grid resident at once; work-groups i and i + snake share a CU) the
// order is mirrored on every second lap of `snake` work-groups, pairing long and short contexts
// on each CU.  Every thread of the work-group must call it (it synchronises).
template <int THREADS>
__device__ __forceinline__ int2 longest_first_unit(const int32_t* context_lens, int n, int hkv, int snake,
                                                   int* len, int* order) {
  for (int t = threadIdx.x; t < n; t += THREADS) len[t] = load_invariant(context_lens + t);
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += THREADS) {
    const int lt = len[t];
    int r = 0;
    for (int u = 0; u < n; ++u) {
      const int lu = len[u];
      r += (lu > lt) | ((lu == lt) & (u < t));
    }
    order[r] = t;
  }
  __syncthreads();
  int j = blockIdx.z * hkv + blockIdx.x;
  if (snake > 0) {
    const int lap = j / snake, pos = j % snake;
    const int lap_len = min(snake, n * hkv - lap * snake);
    if (lap & 1) j = lap * snake + (lap_len - 1 - pos);
  }
  return make_int2(order[j / hkv], j % hkv);
}

}  // namespace pa
