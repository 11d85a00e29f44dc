// Quantization of one page record by one wave64, shared by the prefill and
// append kernels and by the fused decode step (gfx950).
//
// One wave64 quantizes one (page of 32 tokens, KV head):
//  * Key statistics per channel over the page's tokens ("Kitty -- Dynamic
//    Channel-wise Mixed-Precision Keys", How it works / Prefill phase, step 1):
//    a fixed balanced pairwise tree sum for the mean and for the sum of
//    squared deviations m2, exact min and max.  Lane l owns channels 2l, 2l+1
//    and holds all 32 tokens in registers, so the tree is register-local.
//  * Dynamic Channel-wise Precision Boost ("Kitty: Accurate and Efficient
//    2-bit KV Cache Quantization with Dynamic Channel-wise Precision Boost",
//    Abstract; Prefill step 2): the n_hi channels with the largest m2, ties to
//    the lower channel index.  The n_hi-th largest m2 is found by a 31-step
//    bitwise search with wave ballots (m2 >= 0, so its bit pattern orders like
//    the value); equal keys are ranked by channel index with ballot popcounts.
//  * In the running ranking mode the boosted channels come from outside the
//    page instead (the head's exact running variance; see select_top and
//    the running-sum helpers below).
//  * Asymmetric min/max codes (Prefill step 3): hi_bit on boosted channels,
//    lo_bit elsewhere, fp16 step, round-half-even, clamp; split into the base
//    plane (top lo_bit bits) and the boost plane (low lo_bit bits of boosted
//    channels).  BITS = lo_bit: 2 (hi_bit 4) or 4 (hi_bit 8, the last row of
//    the table "Tuning avg_bits").
//  * Values: per token, groups of 32 channels, lo_bit.  Each (token, group)
//    step is formed once, by the lane that loads that group's 64 bytes
//    (packed fp16 min/max); the steps go through LDS to the lanes that code
//    channels c and c + 16 of every token and pack the value words.
//  * Key codes are staged in LDS as bytes and packed into the record's code
//    words with coalesced 16-byte stores.
//
// The fp16 keys are loaded, and the record's code planes and key metadata
// stored, with non-temporal hints: each is touched once, and on gfx950 the
// hint raises the read-and-write stream of this traffic from 0.66 to 0.71
// of the HBM peak.
//
// All float32 arithmetic here is separately rounded (no contraction); the
// step's quotient and reciprocal are the correctly rounded ones, formed
// without a division instruction (see make_step); fp32 -> fp16 conversion
// rounds to nearest even.  Signed zeros of the inputs are read as +0.
#pragma once

#include <type_traits>

#include "kitty_internal.h"

namespace kitty {
namespace pq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Per-wave LDS: Key base codes [32 tokens][128] (4 KB), Key boost codes
// [32][n_hi + 8] (a row per token; column n_hi takes the stores of lanes
// with no boosted channel, so every lane stores unconditionally), value
// steps (1 / step, min) [4 groups][32 tokens] (1 KB).
__host__ __device__ constexpr int boost_row(int n_hi) { return n_hi + 8; }
__host__ __device__ constexpr int lds_vstep(int n_hi) { return 4096 + 32 * boost_row(n_hi); }
__host__ __device__ constexpr int quant_lds_bytes(int n_hi) { return lds_vstep(n_hi) + 1024; }
constexpr int kWaveLds = quant_lds_bytes(128);  // enough for every n_hi

__device__ __forceinline__ float h2f(uint16_t bits) { return (float)__builtin_bit_cast(_Float16, bits); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
// two fp16 inputs with -0 mapped to +0 (x + 0 rounds -0 to +0 and leaves
// every other value unchanged)
__device__ __forceinline__ half2v canon2(uint32_t w) {
  const half2v z = {(_Float16)0.0f, (_Float16)0.0f};
  return __builtin_bit_cast(half2v, w) + z;
}
__device__ __forceinline__ half2v hmin2(half2v a, half2v b) { return __builtin_elementwise_min(a, b); }
__device__ __forceinline__ half2v hmax2(half2v a, half2v b) { return __builtin_elementwise_max(a, b); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// reductions over the 16 lanes of a DPP row: quad xor 1, quad xor 2, half mirror, row mirror
__device__ __forceinline__ float row_min16(float v) {
  v = fminf(v, dpp<0xB1>(v));
  v = fminf(v, dpp<0x4E>(v));
  v = fminf(v, dpp<0x141>(v));
  v = fminf(v, dpp<0x140>(v));
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return v;
}

// Make this wave's LDS writes visible to its later LDS reads by other lanes:
// wait until the writes have completed (measured on gfx950: a ds_read_b128
// issued right after a ds_write_b128 of the same wave can return stale data)
// and keep the compiler from moving memory accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Balanced pairwise tree over 32 values, level by level: a'_i = a_2i + a_2i+1.
__device__ __forceinline__ float tree32(float (&a)[32]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int s = 16; s >= 1; s >>= 1) {
#pragma unroll
    for (int i = 0; i < s; ++i) a[i] = a[2 * i] + a[2 * i + 1];
  }
  return a[0];
}

// The same tree from its second level: a holds the 16 first-level sums.
__device__ __forceinline__ float tree16(float (&a)[32]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1) {
#pragma unroll
    for (int i = 0; i < s; ++i) a[i] = a[2 * i] + a[2 * i + 1];
  }
  return a[0];
}

struct Step {
  float inv;     // 1 / step, or 0 for a zero step
  uint16_t s16;  // fp16 step
};

// Step of the range [mn, mx] over `levels` (L = 3, 15 or 255; inv_levels =
// 1 / L rounded to float32): s16 = f16(r / L) with r = mx - mn, and the
// float32 1 / s16, both correctly rounded, without the division sequence:
// * r / L: q0 = r (1 / L), the remainder r - q0 L by an FMA (exact), and
//   q0 + remainder (1 / L) by a second FMA.  This gives the correctly
//   rounded quotient for every float32 r of the binade [1, 2) and each of
//   the three L (checked exhaustively), hence for every finite r >= 0 here
//   (r <= 131008; the steps scale exactly by powers of two, and r = 0 gives
//   0).
// * 1 / s: one Newton step y0 + (1 - s y0) y0, two FMAs, from v_rcp_f32
//   (within 1 ulp) is correctly rounded for every positive finite fp16 s and
//   every y0 within 1 ulp of 1 / s (checked exhaustively).
__device__ __forceinline__ Step make_step(float mn, float mx, float levels, float inv_levels) {
#pragma clang fp contract(off)
  const float r = mx - mn;
  const float q0 = r * inv_levels;
  const float rem = __builtin_fmaf(-q0, levels, r);
  float q = __builtin_fmaf(rem, inv_levels, q0);
  // q is rounded to float32 and then to fp16 (two roundings, as the
  // definition has them): the empty asm keeps the compiler from fusing the
  // FMA and the conversion into one mixed-precision instruction
  asm("" : "+v"(q));
  const uint16_t s16 = f2h(q);
  const float s = h2f(s16);
  const float y0 = __builtin_amdgcn_rcpf(s);
  const float inv = __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0);
  Step st;
  st.s16 = s16;
  st.inv = (s != 0.0f) ? inv : 0.0f;
  return st;
}

// Float32 arithmetic on fp16 inputs without a separate conversion: one
// v_fma_mix_f32 widens the fp16 operand (half HI of a 32-bit word) exactly
// and rounds once, so it gives the value of converting first and then
// subtracting or adding in float32.  (VALU-only inline asm: the compiler
// does not form the mixed-precision FMA from a conversion and an add.)
template <int HI>
__device__ __forceinline__ float sub_h(uint32_t w, float c) {  // (float)half_HI(w) - c
  float r;
  if constexpr (HI) asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(c));
  else asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(c));
  return r;
}
template <int HI>
__device__ __forceinline__ float add_hh(uint32_t a, uint32_t b) {  // (float)half_HI(a) + (float)half_HI(b)
  float r;
  if constexpr (HI) asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
  else asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// clamp(rne((x - mn) * inv), 0, levels) for the fp16 x in half HI of w,
// inserted as byte `byte` of `into`.  t = (x - mn) * inv is >= 0 and finite
// (x >= mn, inv <= 2^24), and min(rne(t), L) = rne(min(t, L)) for an integer
// L, so the clamp goes first and v_cvt_pk_u8_f32 (round half to even,
// saturating to [0, 255]; checked on gfx950) rounds and packs in one
// instruction.  CLAMP false leaves the clamp out, for a step that
// step_bounds_codes accepts.
template <int HI, bool CLAMP = true>
__device__ __forceinline__ uint32_t code_of(uint32_t w, float mn, float inv, float levels, uint32_t byte = 0, uint32_t into = 0) {
#pragma clang fp contract(off)
  float t = sub_h<HI>(w, mn) * inv;
  if constexpr (CLAMP) t = fminf(t, levels);
  return __builtin_amdgcn_cvt_pk_u8_f32(t, byte, into);
}

// True when the fp16 step s16 of make_step is zero or a normal number.
// Then no code needs the clamp: for zero, inv = 0 and t = 0; for a normal
// step, s16 is within 2^-11 (relative) of (max - min) / L, so with x <= max
// t <= L (1 + 2^-11) (1 + 2^-24)^3 < L + 1/2 for every L <= 255, and
// round-to-nearest-even gives at most L.  A subnormal step (rounding error up
// to half its value) and an infinite one (inv = 0 against an infinite
// difference) keep the clamp.
__device__ __forceinline__ bool step_bounds_codes(uint16_t s16) {
  const uint32_t e = s16 & 0x7C00u;
  return (s16 & 0x7FFFu) == 0u || (e != 0u && e != 0x7C00u);
}

// 2-bit code words: element e of combo A sits at bit 16 (e >> 2) + 4 (e & 1)
// + 2 ((e >> 1) & 1), combo B 8 bits higher, so byte 0 holds combo A's
// elements 0..3, byte 1 combo B's, bytes 2 and 3 their elements 4..7; in
// each byte, elements 0 and 1 (4, 5) take the low two bits of its two
// nibbles and elements 2 and 3 (6, 7) the high two.  Four codes held in
// bytes 0..3 of a dword (each <= 3) become their byte of the word with one
// v_dot4_u32_u8, byte weights 1, 16, 4, 64.
constexpr uint32_t kField2 = 0x40041001u;
__device__ __forceinline__ uint32_t field4(uint32_t x) { return __builtin_amdgcn_udot4(x, kField2, 0u, false); }
// code word from combos A, B given as 8 code bytes each (element e in byte
// e, every byte <= 3)
__device__ __forceinline__ uint32_t pack_word(uint64_t a, uint64_t b) {
  return field4((uint32_t)a) | (field4((uint32_t)b) << 8) | (field4((uint32_t)(a >> 32)) << 16) |
         (field4((uint32_t)(b >> 32)) << 24);
}
constexpr uint64_t kLow2 = 0x0303030303030303ull;  // the low two bits of every byte
constexpr uint64_t kLow4 = 0x0F0F0F0F0F0F0F0Full;  // the low four bits of every byte

// 4-bit code words: element e of the word's combo sits at bit 16 (e >> 2) +
// 8 (e & 1) + 4 ((e >> 1) & 1), so byte k of the word (k < 2) holds elements
// k (low nibble) and k + 2 (high nibble), byte 2 + k elements 4 + k and 6 +
// k.  From 8 code bytes (element e in byte e, each <= 15): byte 0 of the
// word is one v_dot4_u32_u8 of the low four bytes with weights 1, 0, 16, 0.
constexpr uint32_t kEvenNib = 0x00100001u, kOddNib = 0x10000100u;  // byte weights (1, 0, 16, 0), (0, 1, 0, 16)
__device__ __forceinline__ uint32_t nib2(uint32_t x, uint32_t w) { return __builtin_amdgcn_udot4(x, w, 0u, false); }
__device__ __forceinline__ uint32_t pack_word4(uint64_t a) {
  const uint32_t lo = (uint32_t)a, hi = (uint32_t)(a >> 32);
  return nib2(lo, kEvenNib) | (nib2(lo, kOddNib) << 8) | (nib2(hi, kEvenNib) << 16) | (nib2(hi, kOddNib) << 24);
}

// ---- Top-n selection ------------------------------------------------------
// Lane l holds the keys of channels 2l and 2l + 1 (unsigned; a larger key is
// a more sensitive channel).  Selects the n largest keys, ties to the lower
// channel index: the n-th largest key T is found bit by bit with wave
// ballots (TOPBIT = the highest bit a key can have), then the keys equal to
// T are taken in channel order by ballot popcounts.  The search stops early
// once exactly n keys are >= the threshold found so far: the lower bits can
// then only raise it to the n-th key itself, and the keys >= it stay the same
// n (all of them are selected below, ties included).
template <typename K, int TOPBIT>
__device__ __forceinline__ void select_top(K k0, K k1, int n, int lane, bool& h0, bool& h1, int top = TOPBIT) {
  const uint64_t below = (1ull << lane) - 1ull;
  K T = 0;
  int cnt_t = 2 * 64;  // keys >= T: every key is >= 0
  for (int bit = top; bit >= 0 && cnt_t != n; --bit) {  // bits above `top` are clear in every key
    const K cand = T | ((K)1 << bit);
    const int cnt = __popcll(__ballot(k0 >= cand)) + __popcll(__ballot(k1 >= cand));
    if (cnt >= n) {
      T = cand;
      cnt_t = cnt;
    }
  }
  const int gt = __popcll(__ballot(k0 > T)) + __popcll(__ballot(k1 > T));
  const uint64_t e0 = __ballot(k0 == T), e1 = __ballot(k1 == T);
  const int before0 = __popcll(e0 & below) + __popcll(e1 & below);
  const int before1 = before0 + (int)((e0 >> lane) & 1ull);
  const int need = n - gt;
  h0 = (k0 > T) || (k0 == T && before0 < need);
  h1 = (k1 > T) || (k1 == T && before1 < need);
}

// ---- Running sums (the "running" ranking mode) ---------------------------
// "Kitty -- Dynamic Channel-wise Mixed-Precision Keys", How it works:
// Prefill step 1 ranks a head's channels by their variance over the prefill
// sequence, step 5 starts running sums of k and k^2, Decode phase steps 1-2
// update them per token and re-derive the ranking from
// sum k^2 / n - (sum k / n)^2.  The sums are kept exactly: a = k * 2^24 is
// an integer for every finite fp16 k (|a| < 2^40), s1 = sum a in int64,
// s2 = sum a^2 in 128 bits, and the score n s2 - s1^2 (n^2 times that
// variance, in units of 2^-48) is exact, so no accumulation order matters.
typedef unsigned __int128 u128;

// State of one (sequence, KV head), kStatsBytes bytes: two copies of the
// sums, copy c at byte kStatsCopy * c, each int64 s1[128], uint64 s2 low
// halves [128], uint64 s2 high halves [128]; then uint32 mask[4] (channel c
// at bit c & 31 of word c >> 5: the ranking of the last prefill) and
// reserved bytes.  A sequence holding n tokens keeps its sums in copy n & 1,
// so the step that appends token n reads copy n & 1 and writes copy
// (n + 1) & 1 while other waves of the same launch still read copy n & 1.
// Lane l's channels 2l, 2l + 1 are 16 contiguous bytes of each array.
constexpr int kStatsS1 = 0, kStatsS2Lo = 1024, kStatsS2Hi = 2048, kStatsCopy = 3072;
constexpr int kStatsMask = 2 * kStatsCopy, kStatsBytes = kKeyStatsBytes;
static_assert(kStatsMask + 16 <= kStatsBytes, "key statistics layout");
__device__ __forceinline__ uint8_t* sums_copy(uint8_t* st, uint32_t n) { return st + kStatsCopy * (n & 1u); }

// s1 += a, s2 += a^2 for a = k * 2^24 (k the fp16 value with bits h16),
// without a wide multiply: |a| =
// M 2^s with M < 2^11, so a^2 = (M M) 2^(2s) is one 24-bit product shifted
// into 128 bits (below 2^80; its high word is nonzero only for 2s > 42).
__device__ __forceinline__ void accumulate(uint32_t h16, int64_t& s1, u128& s2) {
  const uint32_t e = (h16 >> 10) & 31u, m = h16 & 1023u;
  const uint32_t M = e ? (m | 1024u) : m;
  const uint32_t s = e ? e - 1u : 0u;
  const int64_t a = (int64_t)((uint64_t)M << s);
  s1 += (h16 & 0x8000u) ? -a : a;
  const uint64_t mm = (uint64_t)(M * M);
  const uint32_t sh = 2 * s;
  const uint64_t hi = sh > 42 ? (mm >> (64 - sh)) : 0ull;
  s2 += ((u128)hi << 64) | (mm << sh);
}
// n s2 - s1^2 >= 0 (Cauchy-Schwarz); below 2^127 for n < 2^23
__device__ __forceinline__ u128 running_score(int64_t s1, u128 s2, uint32_t n) {
  const uint64_t m = s1 < 0 ? 0ull - (uint64_t)s1 : (uint64_t)s1;
  return (u128)n * s2 - (u128)m * m;
}

// Lane l's part of a state: the sums of channels 2l, 2l + 1.
struct LaneSums {
  int64_t s1[2];
  u128 s2[2];
};
__device__ __forceinline__ LaneSums load_sums(const uint8_t* st, int lane) {
  typedef int64_t i64x2 __attribute__((ext_vector_type(2)));
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  const i64x2 a = *reinterpret_cast<const i64x2*>(st + kStatsS1 + 16 * lane);
  const u64x2 lo = *reinterpret_cast<const u64x2*>(st + kStatsS2Lo + 16 * lane);
  const u64x2 hi = *reinterpret_cast<const u64x2*>(st + kStatsS2Hi + 16 * lane);
  LaneSums r;
  r.s1[0] = a[0];
  r.s1[1] = a[1];
  r.s2[0] = ((u128)hi[0] << 64) | lo[0];
  r.s2[1] = ((u128)hi[1] << 64) | lo[1];
  return r;
}
__device__ __forceinline__ void store_sums(uint8_t* st, int lane, const LaneSums& r) {
  typedef int64_t i64x2 __attribute__((ext_vector_type(2)));
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<i64x2*>(st + kStatsS1 + 16 * lane) = i64x2{r.s1[0], r.s1[1]};
  *reinterpret_cast<u64x2*>(st + kStatsS2Lo + 16 * lane) = u64x2{(uint64_t)r.s2[0], (uint64_t)r.s2[1]};
  *reinterpret_cast<u64x2*>(st + kStatsS2Hi + 16 * lane) = u64x2{(uint64_t)(r.s2[0] >> 64), (uint64_t)(r.s2[1] >> 64)};
}
// add one token (channels 2l, 2l + 1 as the fp16 pair `k2`, low half first)
__device__ __forceinline__ void add_token(LaneSums& r, uint32_t k2) {
  accumulate(k2 & 0xFFFFu, r.s1[0], r.s2[0]);
  accumulate(k2 >> 16, r.s1[1], r.s2[1]);
}

// Boosted channels given from outside the page (the running mode) or, when
// `given` is false, ranked by the page's own m2.
struct RankIn {
  bool given, h0, h1;
};
// The running ranking over n tokens from lane sums.  The bitwise search
// starts at the highest bit set in any score (a wave maximum), which skips
// most of the 128-bit range.
__device__ __forceinline__ RankIn running_rank(const LaneSums& r, uint32_t n, int n_hi, int lane) {
  RankIn rk{true, false, false};
  if (n_hi >= kHeadDim) {
    rk.h0 = rk.h1 = true;
  } else if (n_hi > 0) {
    const u128 k0 = running_score(r.s1[0], r.s2[0], n), k1 = running_score(r.s1[1], r.s2[1], n);
    const u128 m = k0 > k1 ? k0 : k1;
    const uint64_t mh = (uint64_t)(m >> 64), ml = (uint64_t)m;
    int top = mh ? 127 - __builtin_clzll(mh) : (ml ? 63 - __builtin_clzll(ml) : 0);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) top = max(top, __shfl_xor(top, s));
    select_top<u128, 127>(k0, k1, n_hi, lane, rk.h0, rk.h1, top);
  }
  return rk;
}
// RankIn of lane l's channels from a stored mask (uint32[4])
__device__ __forceinline__ RankIn rank_from_mask(const uint8_t* st, int lane) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(st + kStatsMask)[lane >> 4];
  return RankIn{true, ((w >> ((2 * lane) & 31)) & 1u) != 0, ((w >> ((2 * lane + 1) & 31)) & 1u) != 0};
}

// token t -> value metadata index kappa (inverse of tau): tokens t and
// t + 16 (t < 16) sit at kappa 2t and 2t + 1
__host__ __device__ constexpr int kappa_of(int t) { return 2 * (t & 15) + (t >> 4); }
// (w, e) -> token, kappa = 8w + e
__host__ __device__ constexpr int tau_of(int w, int e) { return 4 * w + (e >> 1) + 16 * (e & 1); }

// Rows of one page: row t at base + t * 128, except that row 31 comes from
// `last` when it is set (the token being appended).
struct RowSrc {
  const _Float16* base;
  const _Float16* last;
  __device__ __forceinline__ const _Float16* row(int t) const {
    return (t == kPageTokens - 1 && last) ? last : base + (size_t)t * kHeadDim;
  }
};

// The Key half of a (page, head) record: statistics, ranking, codes, the two
// code planes and the Key metadata.  Called by a full wave; uses the first
// lds_vstep(NHI) bytes of `lds`.  BITS = lo_bit: 2 (hi 4 / lo 2) or 4
// (hi 8 / lo 4).  n (wave-uniform) channels are boosted, NHI - 16 < n <= NHI:
// the record has NHI boost slots, and slots n .. NHI - 1 hold code 0 and
// index 0.
template <int NHI, int BITS = 2>
__device__ __forceinline__ void quantize_keys_wave(RowSrc ks, uint8_t* __restrict__ rec, uint8_t* __restrict__ lds,
                                                   int n = NHI, RankIn rk = RankIn{false, false, false}) {
#pragma clang fp contract(off)
  static_assert(BITS == 2 || BITS == 4, "lo_bit 2 or 4");
  constexpr float kLo = (float)((1 << BITS) - 1), kHi = (float)((1 << (2 * BITS)) - 1);
  const int lane = threadIdx.x & 63;
  uint8_t* lds_base = lds;          // [32 tokens][128 channels] base codes
  uint8_t* lds_boost = lds + 4096;  // [32 tokens][boost_row(NHI)] boost codes
  wave_lds_sync();

  // ---------------- Key statistics: channels 2*lane, 2*lane + 1 -----------
  // min / max on the fp16 inputs, sums in float32.  A zero extreme may come
  // out as -0 whatever the order, so the extremes are made canonical once at
  // the end (-0 -> +0); the sums need no canonical zeros: a -0 input changes
  // neither m2 nor a code.
  uint32_t xw[32];  // the fp16 pair (channels 2 lane, 2 lane + 1) of each token
  half2v kmn, kmx;
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    xw[t] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ks.row(t) + 2 * lane));
    const half2v hv = __builtin_bit_cast(half2v, xw[t]);
    kmn = t == 0 ? hv : hmin2(kmn, hv);
    kmx = t == 0 ? hv : hmax2(kmx, hv);
  }
  kmn = canon2(__builtin_bit_cast(uint32_t, kmn));
  kmx = canon2(__builtin_bit_cast(uint32_t, kmx));
  const float mn0 = (float)kmn[0], mx0 = (float)kmx[0], mn1 = (float)kmn[1], mx1 = (float)kmx[1];

  // ---------------- Ranking: top n by m2, ties to the lower channel ---------
  // (or the boosted channels given by the running ranking)
  const uint64_t below = (1ull << lane) - 1ull;
  bool h0, h1;
  if (rk.given) {
    h0 = rk.h0;
    h1 = rk.h1;
  } else if (NHI == 0) {
    h0 = h1 = false;
  } else if (NHI == kHeadDim && n == kHeadDim) {
    h0 = h1 = true;
  } else {
    // the tree's first level adds the fp16 inputs pairwise (tokens 2i, 2i + 1)
    float a[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = add_hh<0>(xw[2 * i], xw[2 * i + 1]);
    const float mu0 = tree16(a) * (1.0f / 32.0f);
#pragma unroll
    for (int t = 0; t < 32; ++t) { float d = sub_h<0>(xw[t], mu0); a[t] = d * d; }
    const float m2_0 = tree32(a);
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = add_hh<1>(xw[2 * i], xw[2 * i + 1]);
    const float mu1 = tree16(a) * (1.0f / 32.0f);
#pragma unroll
    for (int t = 0; t < 32; ++t) { float d = sub_h<1>(xw[t], mu1); a[t] = d * d; }
    const float m2_1 = tree32(a);
    // m2 >= 0: its bit pattern orders like its value (bit 31 is clear)
    select_top<uint32_t, 30>(__builtin_bit_cast(uint32_t, m2_0), __builtin_bit_cast(uint32_t, m2_1), n, lane, h0, h1);
  }
  const uint64_t H0 = __ballot(h0), H1 = __ballot(h1);
  const int pos0 = __popcll(H0 & below) + __popcll(H1 & below);
  const int pos1 = pos0 + (h0 ? 1 : 0);

  // ---------------- Key codes and metadata ---------------------------------
  const float L0 = h0 ? kHi : kLo, L1 = h1 ? kHi : kLo;
  constexpr float kInvLo = 1.0f / kLo, kInvHi = 1.0f / kHi;
  const Step st0 = make_step(mn0, mx0, L0, h0 ? kInvHi : kInvLo), st1 = make_step(mn1, mx1, L1, h1 ? kInvHi : kInvLo);
  constexpr float kBoostScale = (float)(1 << BITS);  // kscale = 2^lo_bit * step on boosted channels
  const uint16_t ks0 = h0 ? f2h(kBoostScale * h2f(st0.s16)) : st0.s16;
  const uint16_t ks1 = h1 ? f2h(kBoostScale * h2f(st1.s16)) : st1.s16;
  __builtin_nontemporal_store((uint32_t)ks0 | ((uint32_t)ks1 << 16), reinterpret_cast<uint32_t*>(rec + off_kscale(NHI, BITS) + 4 * lane));
  __builtin_nontemporal_store((uint32_t)f2h(mn0) | ((uint32_t)f2h(mn1) << 16), reinterpret_cast<uint32_t*>(rec + off_kmin(NHI, BITS) + 4 * lane));
  // (pos < n always holds: exactly n channels are selected)
  const bool w0 = h0 && pos0 < NHI, w1 = h1 && pos1 < NHI;
  if (NHI > 0) {
    if (w0) rec[off_idx(NHI, BITS) + pos0] = (uint8_t)(2 * lane);
    if (w1) rec[off_idx(NHI, BITS) + pos1] = (uint8_t)(2 * lane + 1);
    if (lane >= n && lane < NHI) rec[off_idx(NHI, BITS) + lane] = 0;  // padding slots (n < NHI)
    if (lane + 64 >= n && lane + 64 < NHI) rec[off_idx(NHI, BITS) + lane + 64] = 0;
  }
  // Codes go to LDS as bytes: base = q >> BITS on a boosted channel, q
  // elsewhere (BITS bits); boost = q, of which only the low BITS bits are
  // read back.
  const uint32_t sh0 = h0 ? (uint32_t)BITS : 0u, sh1 = h1 ? (uint32_t)BITS : 0u;
  uint8_t* const bst0 = lds_boost + (w0 ? pos0 : NHI);  // column NHI: a lane's discarded stores
  uint8_t* const bst1 = lds_boost + (w1 ? pos1 : NHI);
  // (two copies of the loop: without the clamp when every step of the wave
  // allows it, the usual case, and with it)
  auto key_codes = [&](auto clamp_c) {
    constexpr bool kClamp = decltype(clamp_c)::value;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const uint32_t q = code_of<1, kClamp>(xw[t], mn1, st1.inv, L1, 1, code_of<0, kClamp>(xw[t], mn0, st0.inv, L0));  // bytes q0, q1
      // exactly BITS bits per byte (the planes are packed without masking)
      const uint32_t base = __builtin_amdgcn_ubfe(q, sh0, BITS) | (__builtin_amdgcn_ubfe(q, 8 + sh1, BITS) << 8);
      *reinterpret_cast<uint16_t*>(lds_base + t * 128 + 2 * lane) = (uint16_t)base;
      if (NHI > 0) {
        bst0[t * boost_row(NHI)] = (uint8_t)q;
        bst1[t * boost_row(NHI)] = (uint8_t)(q >> 8);
      }
    }
  };
  if (__ballot(!(step_bounds_codes(st0.s16) && step_bounds_codes(st1.s16))) == 0ull) key_codes(std::false_type{});
  else key_codes(std::true_type{});

  // ---------------- Pack Key code planes from LDS ---------------------------
  wave_lds_sync();
  {
    const int u = lane & 15, w = lane >> 4;
    if (BITS == 2) {
      u32x4 words;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint64_t A = *reinterpret_cast<const uint64_t*>(lds_base + u * 128 + 32 * x + 8 * w);
        const uint64_t B = *reinterpret_cast<const uint64_t*>(lds_base + (16 + u) * 128 + 32 * x + 8 * w);
        words[x] = pack_word(A, B);
      }
      __builtin_nontemporal_store(words, reinterpret_cast<u32x4*>(rec + 16 * lane));
    } else {  // 4-bit: a 32-byte chunk, combo A at word 2x, combo B at 2x + 1
      u32x4 lo, hi;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint64_t A = *reinterpret_cast<const uint64_t*>(lds_base + u * 128 + 32 * x + 8 * w);
        const uint64_t B = *reinterpret_cast<const uint64_t*>(lds_base + (16 + u) * 128 + 32 * x + 8 * w);
        const uint32_t wa = pack_word4(A), wb = pack_word4(B);
        if (x < 2) {
          lo[2 * x] = wa;
          lo[2 * x + 1] = wb;
        } else {
          hi[2 * x - 4] = wa;
          hi[2 * x - 3] = wb;
        }
      }
      __builtin_nontemporal_store(lo, reinterpret_cast<u32x4*>(rec + 32 * lane));
      __builtin_nontemporal_store(hi, reinterpret_cast<u32x4*>(rec + 32 * lane + 16));
    }
    if (NHI > 0) {
      constexpr int nf = NHI / 32;
      uint8_t* const bp = rec + off_kboost(BITS);
      // slots s >= n are padding: their LDS bytes were never written and
      // pack as code 0 (a wave-uniform branch, taken only when n < NHI)
      auto keep = [&](int s0) -> uint64_t {
        const int v = n - s0;  // valid slots among s0 .. s0 + 7
        return v >= 8 ? ~0ull : (v <= 0 ? 0ull : (1ull << (8 * v)) - 1ull);
      };
#pragma unroll
      for (int bb = 0; bb < nf; ++bb) {
        uint64_t A = *reinterpret_cast<const uint64_t*>(lds_boost + u * boost_row(NHI) + 32 * bb + 8 * w);
        uint64_t B = *reinterpret_cast<const uint64_t*>(lds_boost + (16 + u) * boost_row(NHI) + 32 * bb + 8 * w);
        if (n < NHI) {
          const uint64_t m = keep(32 * bb + 8 * w);
          A &= m;
          B &= m;
        }
        if (BITS == 2) {
          __builtin_nontemporal_store(pack_word(A & kLow2, B & kLow2), reinterpret_cast<uint32_t*>(bp + 4 * (lane * nf + bb)));
        } else {
          const u32x2 pr = {pack_word4(A & kLow4), pack_word4(B & kLow4)};
          *reinterpret_cast<u32x2*>(bp + 8 * (lane * nf + bb)) = pr;
        }
      }
      if ((NHI % 32) != 0 && lane < 32) {
        uint64_t A = *reinterpret_cast<const uint64_t*>(lds_boost + u * boost_row(NHI) + 32 * nf + 8 * w);
        uint64_t B = *reinterpret_cast<const uint64_t*>(lds_boost + (16 + u) * boost_row(NHI) + 32 * nf + 8 * w);
        if (n < NHI) {
          const uint64_t m = keep(32 * nf + 8 * w);
          A &= m;
          B &= m;
        }
        if (BITS == 2) {
          *reinterpret_cast<uint32_t*>(bp + 256 * nf + 4 * lane) = pack_word(A & kLow2, B & kLow2);
        } else {
          const u32x2 pr = {pack_word4(A & kLow4), pack_word4(B & kLow4)};
          *reinterpret_cast<u32x2*>(bp + 512 * nf + 8 * lane) = pr;
        }
      }
    }
  }
}

// The Value half of a (page, head) record: per-token steps and minima of
// each group of 32 channels, and the lo_bit codes.  Called by a full wave;
// uses bytes [lds_vstep(NHI), quant_lds_bytes(NHI)) of `lds`, so a Key wave
// and a Value wave can share one area.
template <int NHI, int BITS = 2>
__device__ __forceinline__ void quantize_values_wave(RowSrc vs, uint8_t* __restrict__ rec, uint8_t* __restrict__ lds) {
#pragma clang fp contract(off)
  constexpr float kLo = (float)((1 << BITS) - 1);
  const int lane = threadIdx.x & 63;
  wave_lds_sync();

  // ---------------- Value steps: one (token, group) per lane and pass -------
  bool bounded = true;  // every step of this lane allows codes without the clamp
  {
    float* vstep = reinterpret_cast<float*>(lds + lds_vstep(NHI));  // [group][token] x (1 / step, min)
    uint16_t* vsc = reinterpret_cast<uint16_t*>(rec + off_vscale(NHI, BITS));
    uint16_t* vmn = reinterpret_cast<uint16_t*>(rec + off_vmin(NHI, BITS));
    const int gp = lane & 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tp = (lane >> 2) + 16 * i;
      const u32x4* src = reinterpret_cast<const u32x4*>(vs.row(tp) + 32 * gp);
      u32x4 c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = src[k];
      // (each element is copied to a scalar first: a bit cast of a vector
      // element expression would read the vector's first element)
      const uint32_t w00 = c[0][0];
      half2v mnv = __builtin_bit_cast(half2v, w00), mxv = mnv;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k == 0) continue;
        const uint32_t wk = c[k >> 2][k & 3];
        const half2v h = __builtin_bit_cast(half2v, wk);
        mnv = hmin2(mnv, h);
        mxv = hmax2(mxv, h);
      }
      // zero extremes made canonical once (-0 -> +0), as for the keys
      mnv = canon2(__builtin_bit_cast(uint32_t, mnv));
      mxv = canon2(__builtin_bit_cast(uint32_t, mxv));
      const float mn = fminf((float)mnv[0], (float)mnv[1]);
      const float mx = fmaxf((float)mxv[0], (float)mxv[1]);
      const Step st = make_step(mn, mx, kLo, 1.0f / kLo);
      bounded = bounded && step_bounds_codes(st.s16);
      *reinterpret_cast<float2*>(vstep + 2 * (32 * gp + tp)) = make_float2(st.inv, mn);
      const int kap = kappa_of(tp);
      vsc[32 * gp + kap] = st.s16;
      vmn[32 * gp + kap] = f2h(mn);
    }
  }
  wave_lds_sync();

  // ---------------- Value codes: channels c0 = 32g + u and c0 + 16 ----------
  {
    const int g = lane >> 4, u = lane & 15;
    const int c0 = 32 * g + u, c1 = c0 + 16;
    const floatx4* vstep = reinterpret_cast<const floatx4*>(lds + lds_vstep(NHI)) + 16 * g;  // two tokens per read
    // (each code loop in two copies, as for the keys: without the clamp when
    // every step of the page allows it)
    const bool clamp = __ballot(!bounded) != 0ull;
    if constexpr (BITS == 2) {
      // Element e of word w (token tau(w, e)) goes to byte e & 3 of field
      // f[w][2 (e >> 2) + combo], which is byte 2 (e >> 2) + combo of the
      // word (field4 packs a field's four codes).
      uint32_t f[4][4] = {};
      auto value_codes = [&](auto clamp_c) {
        constexpr bool kClamp = decltype(clamp_c)::value;
#pragma unroll
        for (int t2 = 0; t2 < 16; ++t2) {
          const floatx4 st2 = vstep[t2];  // (1 / step, min) of tokens 2 t2 and 2 t2 + 1
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int t = 2 * t2 + k, kap = kappa_of(t), w = kap >> 3, e = kap & 7;
            const uint16_t* r = reinterpret_cast<const uint16_t*>(vs.row(t));
            const uint32_t y0 = r[c0], y1 = r[c1];
            uint32_t& fa = f[w][2 * (e >> 2)];
            uint32_t& fb = f[w][2 * (e >> 2) + 1];
            fa = code_of<0, kClamp>(y0, st2[2 * k + 1], st2[2 * k], kLo, e & 3, fa);
            fb = code_of<0, kClamp>(y1, st2[2 * k + 1], st2[2 * k], kLo, e & 3, fb);
          }
        }
      };
      if (clamp) value_codes(std::true_type{});
      else value_codes(std::false_type{});
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t word = field4(f[w][0]) | (field4(f[w][1]) << 8) | (field4(f[w][2]) << 16) | (field4(f[w][3]) << 24);
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(rec + off_v(NHI, BITS) + 16 * (16 * w + u) + 4 * g));
      }
    } else {  // 4-bit: combo A (channel c0) at word 2g, combo B (c1) at 2g + 1 of a 32-byte chunk
      uint32_t a0[32], a1[32];
      auto value_codes = [&](auto clamp_c) {
        constexpr bool kClamp = decltype(clamp_c)::value;
#pragma unroll
        for (int t2 = 0; t2 < 16; ++t2) {
          const floatx4 st2 = vstep[t2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int t = 2 * t2 + k;
            const uint16_t* r = reinterpret_cast<const uint16_t*>(vs.row(t));
            a0[t] = code_of<0, kClamp>(r[c0], st2[2 * k + 1], st2[2 * k], kLo);
            a1[t] = code_of<0, kClamp>(r[c1], st2[2 * k + 1], st2[2 * k], kLo);  // codes <= 15: no masking needed below
          }
        }
      };
      if (clamp) value_codes(std::true_type{});
      else value_codes(std::false_type{});
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t wa = 0, wb = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = tau_of(w, e);
          const int sh = 16 * (e >> 2) + 8 * (e & 1) + 4 * ((e >> 1) & 1);
          wa |= a0[t] << sh;
          wb |= a1[t] << sh;
        }
        const u32x2 pr = {wa, wb};
        *reinterpret_cast<u32x2*>(rec + off_v(NHI, BITS) + 32 * (16 * w + u) + 8 * g) = pr;
      }
    }
  }
}

// Quantize and pack one (page, head) into `rec` with one wave; `lds` is this
// wave's private quant_lds_bytes(NHI) bytes; n boosted channels (NHI - 16 <
// n <= NHI).
template <int NHI, int BITS = 2>
__device__ __forceinline__ void quantize_page_wave(RowSrc ks, RowSrc vs, uint8_t* __restrict__ rec, uint8_t* __restrict__ lds,
                                                   int n = NHI, RankIn rk = RankIn{false, false, false}) {
  quantize_keys_wave<NHI, BITS>(ks, rec, lds, n, rk);
  quantize_values_wave<NHI, BITS>(vs, rec, lds);
}


}  // namespace pq
}  // namespace kitty
