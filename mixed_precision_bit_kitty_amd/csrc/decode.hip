// Fused decode attention over the quantized page records (gfx950).
//
// "Kitty: Accurate and Efficient 2-bit KV Cache Quantization with Dynamic
// Channel-wise Precision Boost", Abstract: page dequantization is uniform
// across lanes because each mixed-precision Key page is two uniform 2-bit
// tensors.  Here the dequantization is folded into the two contractions,
//
//   q . k^_t = sum_c (q_c kscale_c) base_tc + sum_j (q_idx_j kscale_idx_j) boost_tj / 4
//              + sum_c q_c kmin_c
//   sum_t p_t v^_tc = sum_t (p_t vscale_t,g) a_tc + sum_t p_t vmin_t,g ,
//
// which run on v_mfma_f32_16x16x32_f16:
//  * codes become exact fp16 operands through the fp4/fp8 conversions: a
//    2-bit code in the low two bits of a nibble is the e2m1 value code / 2
//    (v_cvt_scalef32_pk_f16_fp4 turns a byte's two nibbles into two fp16
//    codes, see fp4_operand), and a 4-bit code of the (hi_bit 8, lo_bit 4)
//    pair in the low nibble of a byte is the e4m3 value code * 2^-9
//    (v_cvt_scalef32_pk_f16_fp8 turns two such bytes into two fp16 codes,
//    see fp8_operand); no code offsets;
//  * the per-page scale goes into the other operand as two fp16 limbs
//    (hi = f16(x), lo = f16(x - hi)), which together carry the product to
//    ~22 bits; the limbs sit in different MFMA rows and are summed after;
//  * the minimum terms are per-page constants that also run on MFMA
//    (constant operands), so no VALU reduction is needed.
//
// One wave = one (sequence, KV head, group of <= 4 query heads, range of
// pages); the last wave of each (sequence, KV head, head group) also attends
// over the fp16 tail page (first, while its first pages load) and takes a
// smaller page range.  Lane l: n = l & 15, w = l >> 4.  QK^T has the query
// limbs as rows (4 head + limb; the other two rows of each head read zeros)
// and the page's tokens as columns, so lane (n, w) ends with the logits of
// head w at tokens n and n + 16; PV has the channels as rows and (head,
// limb) as columns (see decode_kernel).
//
// Pages stream through a per-wave LDS ring with global_load_lds_dwordx4
// (kRing pages in flight); per page the limbs are computed once per
// (head, channel) and per (head, token, group) and exchanged through LDS.
// Online softmax runs in the log2 domain and rescales only when the max
// grows past a slack.  Each wave writes (m, l, O) for its page range; the
// workgroup merges its waves' partials (log-sum-exp), and with several
// workgroups per (sequence, KV head, head group) the last one to arrive
// merges theirs into the output.
#include <type_traits>

#include "kitty_internal.h"
#include "page_quant.h"

namespace kitty {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// The per-page steps are lambdas over the kernel's registers; inlining them
// keeps every operand in VGPRs (an out-of-line call would pass them through
// the stack in scratch memory).
#define KITTY_INLINE __attribute__((always_inline))

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQtHead = kHeadDim + 16;  // padded head row of the q * kscale limbs (halves)
constexpr int kRing = 2;         // pages in flight per wave (LDS DMA streams at full rate with 2)
constexpr int kRowRor4 = 0x124;  // DPP: lane i <- lane (i - 4) mod 16 of its row
constexpr int kRowRor12 = 0x12C; // DPP: lane i <- lane (i + 4) mod 16 of its row

__device__ __forceinline__ floatx4 mfma(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0) only
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// Make this wave's LDS writes visible to its later LDS reads by other lanes:
// wait until the writes have completed (measured on gfx950: a ds_read_b128
// issued right after a ds_write_b128 of the same wave can return stale data)
// and keep the compiler from moving memory accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// MFMA operands from one 2-bit code word.  Element e of combo A sits at bit
// 16 (e >> 2) + 4 (e & 1) + 2 ((e >> 1) & 1), combo B 8 bits higher, so the
// word masked to the low two bits of every nibble (`even`) holds elements
// 0, 1, 4, 5 of both combos in nibbles, and the word shifted right by 2 and
// masked (`odd`) holds elements 2, 3, 6, 7.  A nibble 00cc is the e2m1 value
// c / 2; v_cvt_scalef32_pk_f16_fp4 turns the two nibbles of one byte into two
// fp16 values times `scale` (low nibble into the low half), exactly: scale 2
// gives the code, scale 1/2 the boost weight code / 4.  Three VALU for the
// split and eight conversions for both combos' operands (16 codes).
struct Fp4Word {
  uint32_t even, odd;
};
__device__ __forceinline__ Fp4Word fp4_split(uint32_t w) { return Fp4Word{w & 0x33333333u, (w >> 2) & 0x33333333u}; }
template <int COMBO>
__device__ __forceinline__ half8 fp4_operand(Fp4Word s, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(s.even, scale, COMBO));      // e 0, 1
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(s.odd, scale, COMBO));       // e 2, 3
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(s.even, scale, 2 + COMBO));  // e 4, 5
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(s.odd, scale, 2 + COMBO));   // e 6, 7
  return __builtin_bit_cast(half8, r);
}
typedef __attribute__((address_space(3))) const _Float16 lds_half;  // an fp16 in LDS (32-bit address)
// base + byte K of d in one VALU instruction (an SDWA add with a byte source
// select; the compiler splits it into an extract and an add).  VALU-only
// inline asm.
template <int K>
__device__ __forceinline__ uint32_t add_byte(uint32_t d, uint32_t base) {
  uint32_t r;
  if constexpr (K == 0) asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:DWORD" : "=v"(r) : "v"(d), "v"(base));
  else if constexpr (K == 1) asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD" : "=v"(r) : "v"(d), "v"(base));
  else if constexpr (K == 2) asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD" : "=v"(r) : "v"(d), "v"(base));
  else asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD" : "=v"(r) : "v"(d), "v"(base));
  return r;
}
// MFMA operand from one 4-bit code word (one combo; element e at bit 16 (e
// >> 2) + 8 (e & 1) + 4 ((e >> 1) & 1), so byte k < 2 holds elements k and
// k + 2, byte 2 + k elements 4 + k and 6 + k).  The word masked to the low
// nibble of every byte (`lo`: elements 0, 1, 4, 5) and shifted right by 4
// and masked (`hi`: 2, 3, 6, 7) holds bytes 0000cccc, the e4m3 value c *
// 2^-9 (subnormal for c < 8, normal above, linear across the boundary);
// v_cvt_scalef32_pk_f16_fp8 turns a 16-bit half's two bytes into two fp16
// values times `scale` (low byte into the low half), exactly: scale 2^9
// gives the code, 2^5 the boost weight code / 16.  Three VALU and four
// conversions per word.
__device__ __forceinline__ half8 fp8_operand(uint32_t w, float scale) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, scale, false));  // e 0, 1
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, scale, false));  // e 2, 3
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, scale, true));   // e 4, 5
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, scale, true));   // e 6, 7
  return __builtin_bit_cast(half8, r);
}

// One limb of the q * kscale exchange: [head][channel]; the head stride
// (288 B) and the limb stride (1168 B) put the eight 16-byte rows that one QK
// read instruction touches in distinct LDS banks.
struct QtLimb {
  _Float16 h[4][kQtHead];
  _Float16 pad[8];
};

// Per-wave LDS: ring of kRing records, then the limb exchange areas.  After
// its page loop a wave writes its partial (m, l, O per head) over its ring.
template <int NHI, int BITS>
struct alignas(16) Lds {  // 16-byte aligned size: every wave's area keeps 16-byte alignment
  union {
    uint8_t ring[kRing][rec_bytes(NHI, BITS)];
    float part[4][kPartialStride];  // [head][O[128], m, l, pad]: O 16-byte aligned
  };
  // The q * kscale limbs are read before the softmax and the p limbs after
  // it, so the two exchange areas share memory (a wave's LDS accesses run
  // in program order).
  union {
    QtLimb qt[2];  // q * kscale limbs [limb].h[head][channel]
    struct {
      _Float16 pt[4][2][4][32];  // p * vscale limbs [group][limb][head][p_swz(kappa)]
      _Float16 pl[2][4][32];     // p limbs [limb][head][p_swz(kappa)]
    };
  };
  float red[4][4];              // final value-minimum corrections [head][group]
  int flag;                     // workgroup broadcast of the arrival count (wave 0's copy)
};
static_assert(sizeof(float) * 4 * kPartialStride <= kRing * rec_bytes(0), "partial fits over the ring");
constexpr int kLdsPerCu = 160 * 1024;
// After the waves' areas, one row of 128 fp16 zeros shared by the
// workgroup: the MFMA operand rows and columns whose results are not used
// read it.
constexpr int kZeroRowBytes = 256;
static_assert(sizeof(Lds<128, 2>) * kMaxWgWaves + kZeroRowBytes <= kLdsPerCu, "twelve waves' LDS fit one CU (lo_bit 2)");
// Waves whose LDS areas fit one CU: twelve for every 2-bit record, nine to
// twelve for 4-bit records (a twice larger ring).
template <int NHI, int BITS>
constexpr int max_wg_waves() {
  constexpr int w = (kLdsPerCu - kZeroRowBytes) / (int)sizeof(Lds<NHI, BITS>);
  return w < kMaxWgWaves ? w : kMaxWgWaves;
}
static_assert(max_wg_waves<128, 4>() >= 8, "4-bit records keep two waves per SIMD");

template <int NHI, int BITS>
constexpr int dma_per_page() { return (rec_bytes(NHI, BITS) + 1023) / 1024; }

// Copy one record into an LDS slot: 16 bytes per lane per instruction.  The
// instruction offset advances the global and the LDS address alike, so one
// address serves the 1024-byte chunks within the offset field's reach (up to
// 3072); a chunk at 4096 or beyond (n_hi >= 112, or any 4-bit record) takes
// its own address.  AUX is the cache policy: kDmaStream (nt) for the page
// records, which stream through once (measured on gfx950: the non-temporal
// hint raises a read-only record stream from 0.77 to 0.88 of the HBM peak,
// and this kernel by 2.6% at batch 128); 16 (sc1) reads at agent scope,
// past this CU's vector L1, for a record this launch has just written.
template <int AUX, int M, int NCHUNK, int REM>
__device__ __forceinline__ void dma_chunks(const uint8_t* src, uint8_t* slot, int lane) {
  if constexpr (M < NCHUNK) {
    const bool full = M < NCHUNK - 1 || REM == 0;
    if (full || 16 * lane < REM) {
      if constexpr (1024 * M <= 3072)
        __builtin_amdgcn_global_load_lds(src, (lds_void*)slot, 16, 1024 * M, AUX);
      else
        __builtin_amdgcn_global_load_lds(src + 1024 * M, (lds_void*)(slot + 1024 * M), 16, 0, AUX);
    }
    dma_chunks<AUX, M + 1, NCHUNK, REM>(src, slot, lane);
  }
}
constexpr int kDmaStream = 2;  // the nt bit of the cache-policy operand
template <int NHI, int BITS, int AUX = kDmaStream>
__device__ __forceinline__ void dma_record(const uint8_t* __restrict__ rec, uint8_t* slot, int lane) {
  constexpr int rb = rec_bytes(NHI, BITS);
  dma_chunks<AUX, 0, (rb + 1023) / 1024, rb % 1024>(rec + 16 * lane, slot, lane);
}

// Wait until the oldest in-flight page has landed; `ahead` pages were issued after it.
template <int NHI, int BITS>
__device__ __forceinline__ void wait_page(int ahead) {
  constexpr int L = dma_per_page<NHI, BITS>();
  compiler_fence();
  if (ahead >= 1) wait_vmcnt<L>();
  else wait_vmcnt<0>();
  compiler_fence();
}

template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {  // helper for 16-lane row reductions
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_row<0xB1>(v));
  v = fmaxf(v, dpp_row<0x4E>(v));
  v = fmaxf(v, dpp_row<0x141>(v));
  v = fmaxf(v, dpp_row<0x140>(v));
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_row<0xB1>(v);
  v += dpp_row<0x4E>(v);
  v += dpp_row<0x141>(v);
  v += dpp_row<0x140>(v);
  return v;
}

constexpr float kNegBig = -1.0e30f;  // "no token yet": finite, so exp2(-inf - m) = 0 and m - m = 0

struct WaveState {
  float m;        // running max of the scaled logits of head w (log2 domain)
  float l;        // this lane's share of head w's softmax denominator
  floatx4 o[8];   // PV accumulators, channel blocks of 16
  floatx4 corr;   // value-minimum correction accumulator
};

// Value of head (n & 3) from a per-head value held by rows (row h = head h).
__device__ __forceinline__ float head_of_column(float v_row, int n) {
  const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v_row), 0));
  const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v_row), 16));
  const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v_row), 32));
  const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v_row), 48));
  const int hc = n & 3;
  return hc == 0 ? a0 : (hc == 1 ? a1 : (hc == 2 ? a2 : a3));
}

// Online softmax step for lane (n, w): raw logits s0, s1 of head w at tokens
// n and n + 16 of the page; they become probabilities.  The max over the
// page's 32 tokens is a 16-lane row reduction.  The reference m is raised
// only when a logit exceeds it by more than `slack` (log2 units), so after
// the first page a rescale is rare; until then probabilities may reach
// 2^slack.  The fp16 limb hi = f16(p_hi * vscale) is finite while
// p_hi * vscale < 65520: the page's slack is kSlack when every vscale of the
// page is at most kVsSafe (2^8 * 255.5 < 65504), else 0, which keeps p <= 1
// and p * vscale <= vscale <= 43680 (the largest fp16 step of a range of two
// finite fp16 values over 3 levels).  The PV accumulators hold head n & 3 in
// column n, so their rescale factor is read from that head's row.
constexpr float kSlack = 8.0f;
constexpr float kVsSafe = 255.5f;
constexpr uint32_t kVsSafeBits = 0x5BFCu;  // fp16 bits of kVsSafe
static_assert(kVsSafe == 511.0f / 2.0f, "kVsSafe = 255.5: fp16 0x5BFC (exponent 22, mantissa 0x3FC)");
__device__ __forceinline__ void softmax_step(WaveState& st, float& s0, float& s1, float sl2, int n,
                                             float slack = kSlack) {
  const float mx = row_max16(fmaxf(s0, s1)) * sl2;
  if (__ballot(mx > st.m + slack)) {  // wave-uniform
    const float mnew = fmaxf(st.m, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
    st.l *= alpha;
    const float ao = head_of_column(alpha, n);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) st.o[mb] *= ao;
    st.corr *= ao;
    st.m = mnew;
  }
  s0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, sl2, -st.m));
  s1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, sl2, -st.m));
  st.l += s0 + s1;
}

// p limbs (hi = f16(p), lo = f16(p - hi)) of tokens (n, n + 16)
struct PLimbs {
  half2v hi, lo;
};
__device__ __forceinline__ PLimbs p_limbs(float p0, float p1) {
  const half2v hi = {(_Float16)p0, (_Float16)p1};
  // p - hi is exact in fp32; one mixed-precision fma rounds it to fp16
  const half2v lo = {(_Float16)__builtin_fmaf((float)hi[0], -1.0f, p0), (_Float16)__builtin_fmaf((float)hi[1], -1.0f, p1)};
  return PLimbs{hi, lo};
}
// Position of kappa in row r = 4 limb + head of a p-limb table: the 16-byte
// chunk kappa / 8 is XOR-swizzled with (r / 2) mod 4, so the eight rows that
// one PV operand read touches (same chunk) fall in eight distinct 4-bank
// groups instead of two; the half2 writes stay conflict-free.
__device__ __forceinline__ int p_swz(int r, int kappa) { return (((kappa >> 3) ^ ((r >> 1) & 3)) << 3) | (kappa & 7); }
// Write the p limbs of tokens (n, n + 16) of head w at kappa (2n, 2n + 1):
// dst[limb][w][p_swz(4 limb + w, kappa)].
__device__ __forceinline__ void store_p_limbs(_Float16 (*dst)[4][32], int w, int n, PLimbs pl) {
  *reinterpret_cast<half2v*>(&dst[0][w][p_swz(w, 2 * n)]) = pl.hi;
  *reinterpret_cast<half2v*>(&dst[1][w][p_swz(4 + w, 2 * n)]) = pl.lo;
}
// Two fp16 limbs of a * b for fp16 a, b (exact product: 22 significant
// bits): hi = f16(a b) by a correctly rounded fp16 multiply and lo = the
// residual a b - hi, which one fused fp16 multiply-add forms exactly (it has
// at most 11 significant bits) unless it falls below the fp16 normal range.
// Packed: one instruction per limb for two products.
__device__ __forceinline__ half2v mul_hi(half2v a, half2v b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ half2v fma2(half2v a, half2v b, half2v c) { return __builtin_elementwise_fma(a, b, c); }

// Share of the pages given to wave i of a workgroup.  Wave i runs on SIMD
// i % 4 as its (i / 4)-th resident wave, and the instruction arbiter favours
// older waves: with equal shares the youngest class finishes last, running
// alone at the end.  Shares 9 : 7 : 5 measured about 5% faster than equal
// shares on the batch-16, 4096-token decode, and 10 : 7 : 4 about 5% faster
// again once the page records stream with the non-temporal hint.
__host__ __device__ __forceinline__ int page_weight(int i) { return i < 4 ? 10 : (i < 8 ? 7 : 4); }
// Share of the tail wave (the last wave of a unit, wave W - 1 of its last
// workgroup): it streams pages too, after its fp16 tail.
#ifndef KITTY_TAIL_DROP
#define KITTY_TAIL_DROP 2
#endif
__host__ __device__ __forceinline__ int tail_weight(int W) {
  const int t = page_weight(W - 1) - KITTY_TAIL_DROP;
  return t > 0 ? t : 0;
}
// sum of page_weight(j) for j < i (i <= W <= 12)
__host__ __device__ __forceinline__ int weight_prefix(int i, int W) {
  const int r = min(i, W);
  return 10 * min(r, 4) + 7 * min(max(r - 4, 0), 4) + 4 * max(r - 8, 0);
}

// A workgroup of W = wg_waves waves (at most twelve: three per SIMD, with
// registers held to 168 per lane) works on one (sequence, KV head, head
// group); n_wg such workgroups share it.  Each wave keeps its own LDS area.
//
// Lane (n = lane & 15, w = lane >> 4) roles:
//  * QK^T has the query limbs as rows (row r = 4 head + slot, slots 0/1 = hi/lo
//    limb, 2/3 zero) and the tokens as columns, so lane (n, w) ends with
//    the logits of head w at tokens n (combo A) and n + 16 (combo B);
//  * PV has channels as rows and (head n & 3, limb (n >> 2) & 1) as columns
//    0..7, the p limbs for the value-minimum correction as columns 8..15.
// RUN: the fused step in the running ranking mode (p.key_stats set); a
// separate instantiation, so the page mode's kernels carry none of its code.
template <int NHI, int BITS, bool RUN>
__global__ __launch_bounds__(64 * kMaxWgWaves) __attribute__((amdgpu_waves_per_eu(3, 3)))
void decode_kernel(DecodeParams p) {
  constexpr int NB = (NHI + 31) / 32;  // boost slot blocks (the last may be half)
  constexpr int NF = NHI / 32;         // full boost blocks
  constexpr int RB = rec_bytes(NHI, BITS);
  static_assert(BITS == 2 || BITS == 4, "lo_bit 2 or 4");
  static_assert(sizeof(Lds<NHI, BITS>) >= pq::quant_lds_bytes(NHI), "a wave's LDS holds the page quantizer's scratch");
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  Lds<NHI, BITS>* const all = reinterpret_cast<Lds<NHI, BITS>*>(dyn_lds);
  Lds<NHI, BITS>& sm = all[wave];
  _Float16* const zrow = reinterpret_cast<_Float16*>(all + p.wg_waves);  // kZeroRowBytes, 16-byte aligned

  const int W = p.wg_waves;
  const int n_pw = p.n_wg * W - 1;           // the last wave of this unit also takes the tail
  const int pw = blockIdx.x * W + wave;
  const bool tail_wave = pw == n_pw;
  const int hk = blockIdx.y / p.n_head_groups, hg = blockIdx.y % p.n_head_groups;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63, n = lane & 15, w = lane >> 4;
  const int h = n & 3, limb = (n >> 2) & 1;  // PV column role
  const int ah = n >> 2, al = n & 1;         // QK row role (A operand)
  const int hq0 = hk * p.group + 4 * hg;
  const int gcount = min(4, p.group - 4 * hg);

  // Pages [0, Pm) of the longest allowed sequence are divided over the page
  // waves in proportion to page_weight (the older waves of a SIMD get more).
  const int Pm = min(p.max_seq_len / kPageTokens, p.max_pages);
  // (32-bit products: c0 + 10 <= 16 x 84 and Pm <= 4096)
  const int tw = tail_weight(W);
  const int wsum = p.n_wg * weight_prefix(W, W) - page_weight(W - 1) + tw;
  const int c0 = (int)blockIdx.x * weight_prefix(W, W) + weight_prefix(wave, W);
  const int p0 = (c0 * Pm) / wsum;  // the tail wave's range ends at Pm
  const int p1m = ((c0 + (tail_wave ? tw : page_weight(wave))) * Pm) / wsum;
  // Independent loads first (one memory round trip before the first DMA):
  // the sequence length, this wave's page ids (lane j: page p0 + j), queries.
  const size_t page_row = (size_t)b * p.max_pages;
  const int seq_raw = p.seq_lens[b];
  const int id_raw = lane < p1m - p0 ? p.block_table[page_row + p0 + lane] : -1;
  const _Float16* qg = p.q + ((size_t)b * p.n_q_heads + hq0) * kHeadDim;
  half8 bq_plain[4];  // plain q as QK rows 4 head + 0 (the minimum term), zero elsewhere
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    half8 v = {};
    if ((n & 3) == 0 && ah < gcount) v = *reinterpret_cast<const half8*>(qg + ah * kHeadDim + 32 * kb + 8 * w);
    bq_plain[kb] = v;
  }
  // producer of the q * kscale limbs: head ph, channels pc .. pc + 7
  const int ph = lane & 3, pc = 8 * (lane >> 2);
  half8 q_prod = {};
  if (ph < gcount) q_prod = *reinterpret_cast<const half8*>(qg + ph * kHeadDim + pc);
  // The fused step appends one token first: the tail wave stores it (and
  // seals the tail page it fills) before its own attention, while few
  // registers are live; every wave attends as if that append had happened
  // before the call.
  const bool fused = p.k_new != nullptr && seq_raw >= 0;  // a negative length marks an inactive slot
  const int n0 = seq_raw < 0 ? 0 : seq_raw;  // tokens stored before this call
  const int total = fused ? n0 + 1 : n0;
  const size_t toff = ((size_t)b * p.n_kv_heads + hk) * kPageTokens * kHeadDim;  // (b, hk) tail
  const size_t noff = ((size_t)b * p.n_kv_heads + hk) * kHeadDim;  // (b, hk) row of k_new / v_new
  uint8_t* seal_rec = nullptr;  // the record this call sealed (wave-uniform; tail wave only)
  pq::LaneSums run{};  // running mode: the head's sums with the new token
  if (tail_wave && fused) {
    if constexpr (RUN) {
      // running ranking mode ("Kitty -- Dynamic Channel-wise Mixed-Precision
      // Keys", Decode phase steps 1-2): every head group adds the new token to
      // the current copy of the sums; head group 0 stores the result as the
      // next copy, which no wave of this launch reads
      uint8_t* st = p.key_stats + ((size_t)b * p.n_kv_heads + hk) * pq::kStatsBytes;
      run = pq::load_sums(pq::sums_copy(st, (uint32_t)n0), lane);
      pq::add_token(run, *reinterpret_cast<const uint32_t*>(p.k_new + noff + 2 * lane));
      if (hg == 0) pq::store_sums(pq::sums_copy(st, (uint32_t)n0 + 1), lane, run);
    }
    if (hg == 0) {  // the append: the token goes to tail slot n0 mod 32
      const int slot = n0 % kPageTokens;
      *reinterpret_cast<uint32_t*>(p.tail_k + toff + (size_t)slot * kHeadDim + 2 * lane) =
          *reinterpret_cast<const uint32_t*>(p.k_new + noff + 2 * lane);
      *reinterpret_cast<uint32_t*>(p.tail_v + toff + (size_t)slot * kHeadDim + 2 * lane) =
          *reinterpret_cast<const uint32_t*>(p.v_new + noff + 2 * lane);
    }
    const int pg = n0 / kPageTokens;
    const int phys = n0 % kPageTokens == kPageTokens - 1 && pg < p.max_pages ? p.block_table[page_row + pg] : -1;
    if (phys >= 0 && (int64_t)phys < p.n_pages) {  // wave-uniform; else there is no seal (or it is skipped)
      // The filled tail (slots 0..30 and the new token) becomes page n0 / 32,
      // quantized exactly as prefill and append do.  Head group 0 writes the
      // record into the pool; other head groups quantize their own copy into
      // the workspace.
      seal_rec = hg == 0 ? p.pages + (int64_t)phys * p.page_bytes + (int64_t)hk * RB
                         : p.seal_scratch + ((((size_t)b * p.n_kv_heads + hk) * (p.n_head_groups - 1)) +
                                             (hg - 1)) * RB;
      pq::RankIn rk{false, false, false};
      if constexpr (RUN) rk = pq::running_rank(run, (uint32_t)n0 + 1, p.n_hi, lane);
      pq::quantize_page_wave<NHI, BITS>(pq::RowSrc{p.tail_k + toff, p.k_new + noff},
                                        pq::RowSrc{p.tail_v + toff, p.v_new + noff}, seal_rec,
                                        reinterpret_cast<uint8_t*>(&sm), p.n_hi, rk);
    }
  }

  // Tokens attended: the first seq = min(total, max_seq_len).  When the
  // bound falls inside a sealed page (not the sequence's tail page), that
  // page is attended up to the bound (last_lim tokens) and no tail token is.
  const int seq = total > p.max_seq_len ? p.max_seq_len : total;
  const int pfull = seq / kPageTokens;
  const int rem = seq - pfull * kPageTokens;
  const bool part_sealed = rem > 0 && pfull < total / kPageTokens;
  int P = part_sealed ? pfull + 1 : pfull;  // pages attended, the last one possibly in part
  int last_lim = part_sealed ? rem : kPageTokens;
  if (P > p.max_pages) {  // now P <= Pm + 1
    P = p.max_pages;
    last_lim = kPageTokens;
  }
  const int ntail = part_sealed ? 0 : rem;
  // A seal by this call makes page n0 / 32: the tail wave attends it (when
  // its block table entry is valid; else, like any invalid page, it adds
  // nothing) and the page waves leave it out.  The tail wave also takes a
  // sealed page the bound cuts (page pfull, beyond every page wave's range).
  const bool new_page = fused && n0 % kPageTokens == kPageTokens - 1 && P > n0 / kPageTokens;
  const bool extra_page = new_page || (part_sealed && P == pfull + 1);
  const int p1 = min(p1m, extra_page ? P - 1 : P);
  const int npg = p1 > p0 ? p1 - p0 : 0;
  const uint8_t* head_base = p.pages + (int64_t)hk * RB;
  // page ids are int32 and the page stride is below 2^32 (at most 1024 KV
  // heads): id checks and record offsets stay in scalar 32-bit arithmetic
  const int np32 = p.n_pages > 0x7FFFFFFF ? 0x7FFFFFFF : (int)p.n_pages;
  const uint32_t pb32 = (uint32_t)p.page_bytes;
  const int ids = lane < npg ? id_raw : -1;  // physical page of p0 + lane (at most 64 per wave)
  auto phys_of = [&](int i) -> int { return __builtin_amdgcn_readlane(ids, i); };
  auto rec_of = [&](int phys) -> const uint8_t* {
    if (phys < 0 || phys >= np32) phys = 0;  // invalid ids read page 0 and are masked
    return head_base + (uint64_t)(uint32_t)phys * pb32;
  };
  if (seal_rec != nullptr) {  // the ring overlaps the quantizer's LDS scratch: its accesses are done first
    wait_lgkm0();
    compiler_fence();
  }
#pragma unroll
  for (int d = 0; d < kRing; ++d)
    if (d < npg) dma_record<NHI, BITS>(rec_of(phys_of(d)), sm.ring[d], lane);

  // ---- per-wave constants -------------------------------------------------
  // Power-of-two scale of the query in the q * kscale limbs: 2^-qe brings
  // every |q| of the head group to at most 1.49, so that q 2^-qe * kscale
  // stays below 65504 for every kscale the quantizer can produce (at most
  // 43680: the step of a range of two finite fp16 values over 3 levels); the
  // logits are scaled back by 2^qe in fp32, exactly.
  int qe = 0;
  {
    float qa = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) qa = fmaxf(qa, fabsf((float)q_prod[j]));
    qa = row_max16(qa);
    qa = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qa), 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qa), 16))),
               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qa), 32)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qa), 48))));
    for (int i = 0; i < 16 && qa > 1.49f; ++i) {  // wave-uniform; 65504 / 2^16 < 1
      qa *= 0.5f;
      ++qe;
    }
    if (qe) {
      const float f = __builtin_ldexpf(1.0f, -qe);
#pragma unroll
      for (int j = 0; j < 8; ++j) q_prod[j] = (_Float16)((float)q_prod[j] * f);
    }
  }
  const float qsc = __builtin_ldexpf(1.0f, qe);
  const float sl2 = (1.0f / sqrtf((float)kHeadDim)) * kLog2e;
  // PV B operand source: lanes n < 8 read the group's p * vscale limbs, lanes
  // n >= 8 the p limbs (same address for every group)
  const int pk = p_swz(4 * limb + h, 8 * w);  // this lane's operand chunk in its row
  const _Float16* b_src = n < 8 ? &sm.pt[0][limb][h][pk] : &sm.pl[limb][h][pk];
  const int b_stride = n < 8 ? 2 * 4 * 32 : 0;
  // Columns 8..15 of the PV products are not used (only the correction
  // MFMA, which takes group 0's operand, needs the p limbs there): for
  // groups 1..3 those lanes read zeros, which lowers the switching power
  // as the zero QK rows do.
  const _Float16* b_rest = n < 8 ? &sm.pt[0][limb][h][pk] : zrow;

  // every wave writes the zero row (the same zeros) before its own first read
  // of it, which follows its first limb exchange's wait
  *reinterpret_cast<uint32_t*>(&zrow[2 * lane]) = 0u;
  WaveState st;
  st.m = kNegBig;
  st.l = 0.0f;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) st.o[mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  st.corr = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  auto valid_of = [&](int i) {
    const int phys = phys_of(i);
    return phys >= 0 && phys < np32;  // wave-uniform
  };
  // q * kscale limbs of the page in S, one (head, 8 channels) per lane
  auto produce_qt = [&](const uint8_t* S) KITTY_INLINE {
    const half8 ks = *reinterpret_cast<const half8*>(S + off_kscale(NHI, BITS) + 2 * pc);
    half8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const half2v a = {q_prod[j], q_prod[j + 1]}, b = {ks[j], ks[j + 1]};
      const half2v h2 = mul_hi(a, b);
      const half2v l2 = fma2(a, b, -h2);
      hi[j] = h2[0];
      hi[j + 1] = h2[1];
      lo[j] = l2[0];
      lo[j + 1] = l2[1];
    }
    *reinterpret_cast<half8*>(&sm.qt[0].h[ph][pc]) = hi;
    *reinterpret_cast<half8*>(&sm.qt[1].h[ph][pc]) = lo;
  };
  // QK^T of the page in S (its q * kscale limbs in LDS): rows = (head, limb),
  // columns = tokens; the logits of head w at tokens n and n + 16
  // the boosted channels' indices of the page in S (4 per word), read before
  // the limb exchange so that the gathers can follow its barrier at once
  struct BoostIdx {
    u32x2 ib[NB > 0 ? NB : 1];
  };
  auto boost_idx = [&](const uint8_t* S) KITTY_INLINE {
    BoostIdx r;
#pragma unroll
    for (int k2 = 0; k2 < NB; ++k2) {
      const int q0 = 32 * k2 + 8 * w;
      r.ib[k2] = q0 < NHI ? *reinterpret_cast<const u32x2*>(S + off_idx(NHI, BITS) + q0) : u32x2{};
    }
    return r;
  };
  // lim: tokens of the page below the attention bound (32 but for a page the
  // bound cuts)
  // QK operand row of this lane: rows 4 head + 0 / 1 carry the hi / lo limb;
  // rows 4 head + 2 / 3 are not used and read zeros, which lowers the
  // MFMAs' switching power and with it the clock throttling under load
  // (about 2% at batch 128, same results)
  const _Float16* const qrow = (n & 2) ? zrow : sm.qt[al].h[ah];
  auto qk = [&](const uint8_t* S, const BoostIdx& bi, bool valid, int lim, float& s0, float& s1) KITTY_INLINE {
    // this lane's K base chunk: four words (2-bit) or eight (4-bit: combos A, B of word x at 2x, 2x + 1)
    const u32x4 kw = *reinterpret_cast<const u32x4*>(S + 16 * BITS / 2 * lane);
    const u32x4 kw2 = BITS == 4 ? *reinterpret_cast<const u32x4*>(S + 32 * lane + 16) : u32x4{};
    half8 bq[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) bq[kb] = *reinterpret_cast<const half8*>(&qrow[32 * kb + 8 * w]);
    half8 bb[NB > 0 ? NB : 1];
    u32x2 bw[NB > 0 ? NB : 1];  // 2-bit: one word (both combos); 4-bit: the combo A, B pair
#pragma unroll
    for (int k2 = 0; k2 < NB; ++k2) {
      const int q0 = 32 * k2 + 8 * w;
      half8 v = {};
      if (q0 < NHI) {
        // byte offsets 2 idx of the eight channels: the index bytes, taken
        // to their low 7 bits (a channel index is below 128, and the mask
        // keeps every gather inside its 256-byte row whatever the record
        // holds), double without a carry across bytes, and one SDWA add
        // per channel forms its LDS address
        const uint32_t d0 = (bi.ib[k2][0] & 0x7F7F7F7Fu) << 1, d1 = (bi.ib[k2][1] & 0x7F7F7F7Fu) << 1;
        const uint32_t qb = (uint32_t)(uintptr_t)(const lds_half*)qrow;  // LDS byte address
        const uint32_t ad[8] = {add_byte<0>(d0, qb), add_byte<1>(d0, qb), add_byte<2>(d0, qb), add_byte<3>(d0, qb),
                                add_byte<0>(d1, qb), add_byte<1>(d1, qb), add_byte<2>(d1, qb), add_byte<3>(d1, qb)};
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = *(const lds_half*)(uintptr_t)ad[j];
      }
      bb[k2] = v;
      if constexpr (BITS == 2) {
        if (k2 < NF) bw[k2][0] = *reinterpret_cast<const uint32_t*>(S + off_kboost() + 4 * (lane * NF + k2));
        else bw[k2][0] = lane < 32 ? *reinterpret_cast<const uint32_t*>(S + off_kboost() + 256 * NF + 4 * lane) : 0u;
      } else {
        if (k2 < NF) bw[k2] = *reinterpret_cast<const u32x2*>(S + off_kboost(4) + 8 * (lane * NF + k2));
        else bw[k2] = lane < 32 ? *reinterpret_cast<const u32x2*>(S + off_kboost(4) + 512 * NF + 8 * lane) : u32x2{};
      }
    }
    // the gathers (a second LDS round trip after the index read) and, when
    // registers allow (at most two boost blocks), the minimum reads issue
    // with the limb reads, ahead of the MFMAs
    constexpr bool kEarlyMin = NB <= 2;
    auto kmin_of = [&](int kb) { return *reinterpret_cast<const half8*>(S + off_kmin(NHI, BITS) + 2 * (32 * kb + 8 * w)); };
    half8 kmins[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      if constexpr (kEarlyMin) kmins[kb] = kmin_of(kb);
    __builtin_amdgcn_sched_barrier(0);
    floatx4 cmin = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) cmin = mfma(bq_plain[kb], kEarlyMin ? kmins[kb] : kmin_of(kb), cmin);
    floatx4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if constexpr (BITS == 2) {
        const Fp4Word f = fp4_split(kw[kb]);
        acc0 = mfma(bq[kb], fp4_operand<0>(f, 2.0f), acc0);
        acc1 = mfma(bq[kb], fp4_operand<1>(f, 2.0f), acc1);
      } else {
        const uint32_t wa = kb < 2 ? kw[2 * kb] : kw2[2 * kb - 4];
        const uint32_t wb = kb < 2 ? kw[2 * kb + 1] : kw2[2 * kb - 3];
        acc0 = mfma(bq[kb], fp8_operand(wa, 512.0f), acc0);
        acc1 = mfma(bq[kb], fp8_operand(wb, 512.0f), acc1);
      }
    }
#pragma unroll
    for (int k2 = 0; k2 < NB; ++k2) {
      if constexpr (BITS == 2) {
        const Fp4Word f = fp4_split(bw[k2][0]);
        acc0 = mfma(bb[k2], fp4_operand<0>(f, 0.5f), acc0);
        acc1 = mfma(bb[k2], fp4_operand<1>(f, 0.5f), acc1);
      } else {
        acc0 = mfma(bb[k2], fp8_operand(bw[k2][0], 32.0f), acc0);
        acc1 = mfma(bb[k2], fp8_operand(bw[k2][1], 32.0f), acc1);
      }
    }
    // rows 4w (hi limb, with the minimum term) + 4w + 1 (lo limb) of head w;
    // the code terms carry the query scale 2^-qe, the minimum term does not
    const float cst = cmin[0];
    s0 = valid && n < lim ? __builtin_fmaf(acc0[0] + acc0[1], qsc, cst) : -INFINITY;       // token n
    s1 = valid && n + 16 < lim ? __builtin_fmaf(acc1[0] + acc1[1], qsc, cst) : -INFINITY;  // token n + 16
  };
  // p * vscale limbs (tokens n, n + 16 of head w, all four groups) and p
  // limbs.  With p = p_hi + p_lo (fp16 limbs), p * vscale = hi + lo where
  // hi = f16(p_hi vscale), lo = f16(p_lo vscale + (p_hi vscale - hi)): the
  // inner residual is exact and lo is rounded once, so the pair carries
  // p * vscale to about 2^-21 relative.
  // The page's value steps of tokens (2n, 2n + 1) in all four groups (lane
  // (n, w) and its row neighbours read the same; together the lanes cover
  // the page's 128 steps), read before the softmax: their maximum sets the
  // page's slack.
  struct VScales {
    half2v g[4];
  };
  auto read_vscales = [&](const uint8_t* S) KITTY_INLINE {
    VScales v;
#pragma unroll
    for (int g = 0; g < 4; ++g) v.g[g] = *reinterpret_cast<const half2v*>(S + off_vscale(NHI, BITS) + 2 * (32 * g + 2 * n));
    return v;
  };
  auto page_slack = [&](const VScales& v) KITTY_INLINE {
    // steps are >= 0 (and not NaN), so their fp16 bit patterns order like
    // their values: an unsigned maximum and one compare with kVsSafe's bits
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    auto bits = [](half2v x) { return __builtin_bit_cast(u16x2, x); };
    const u16x2 a = __builtin_elementwise_max(__builtin_elementwise_max(bits(v.g[0]), bits(v.g[1])),
                                              __builtin_elementwise_max(bits(v.g[2]), bits(v.g[3])));
    const uint32_t m = a[0] > a[1] ? a[0] : a[1];
    return __ballot(m > kVsSafeBits) ? 0.0f : kSlack;
  };
  auto produce_pt = [&](const VScales& vsc, float s0, float s1) KITTY_INLINE {
    const PLimbs pl = p_limbs(s0, s1);
    const half2v* vsg = vsc.g;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const half2v vs = vsg[g];
      const half2v hi = mul_hi(pl.hi, vs);
      const half2v lo = fma2(pl.lo, vs, fma2(pl.hi, vs, -hi));
      *reinterpret_cast<half2v*>(&sm.pt[g][0][w][p_swz(w, 2 * n)]) = hi;
      *reinterpret_cast<half2v*>(&sm.pt[g][1][w][p_swz(4 + w, 2 * n)]) = lo;
    }
    store_p_limbs(sm.pl, w, n, pl);
  };
  // PV of the page in S (its p limbs in LDS)
  auto pv = [&](const uint8_t* S) KITTY_INLINE {
    const u32x4 vw = *reinterpret_cast<const u32x4*>(S + off_v(NHI, BITS) + 16 * BITS / 2 * lane);
    const u32x4 vw2 = BITS == 4 ? *reinterpret_cast<const u32x4*>(S + off_v(NHI, BITS) + 32 * lane + 16) : u32x4{};
    // columns 0..7: p * vscale limbs of group g; 8..15: p limbs for the
    // correction (group 0), zeros (groups 1..3)
    half8 bgs[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) bgs[g] = *reinterpret_cast<const half8*>(g == 0 ? b_src : b_rest + g * b_stride);
    // correction operand: rows 0..3 the page's vmin of group n; the other
    // rows read zeros (the codes carry no offset)
    const uint8_t* src = n < 4 ? S + off_vmin(NHI, BITS) + 2 * (32 * n + 8 * w) : reinterpret_cast<const uint8_t*>(zrow);
    const half8 a = *reinterpret_cast<const half8*>(src);
    // every operand read is issued before the first MFMA: one LDS round trip
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const half8 bg = bgs[g];
      if constexpr (BITS == 2) {
        const Fp4Word f = fp4_split(vw[g]);
        st.o[2 * g] = mfma(fp4_operand<0>(f, 2.0f), bg, st.o[2 * g]);
        st.o[2 * g + 1] = mfma(fp4_operand<1>(f, 2.0f), bg, st.o[2 * g + 1]);
      } else {
        const uint32_t wa = g < 2 ? vw[2 * g] : vw2[2 * g - 4];
        const uint32_t wb = g < 2 ? vw[2 * g + 1] : vw2[2 * g - 3];
        st.o[2 * g] = mfma(fp8_operand(wa, 512.0f), bg, st.o[2 * g]);
        st.o[2 * g + 1] = mfma(fp8_operand(wb, 512.0f), bg, st.o[2 * g + 1]);
      }
    }
    st.corr = mfma(a, bgs[0], st.corr);
  };
  // one page through the whole contraction
  // (all the page's reads of the record come before the first limb write:
  // the compiler cannot tell those writes from the record, and would
  // otherwise wait for each read)
  auto attend_page = [&](const uint8_t* S, bool valid, int lim) KITTY_INLINE {
    const BoostIdx bi = boost_idx(S);
    const VScales vsc = read_vscales(S);
    produce_qt(S);
    wave_lds_sync();
    float s0, s1;
    qk(S, bi, valid, lim, s0, s1);
    softmax_step(st, s0, s1, sl2, n, page_slack(vsc));
    produce_pt(vsc, s0, s1);
    wave_lds_sync();
    pv(S);
  };

  // With a seal attended, the tail is empty; a seal beyond a smaller
  // max_seq_len leaves the older tail tokens to attend.
  if (tail_wave && ntail > 0 && !new_page) {
    // fp16 tail tokens: the same contraction with fp16 K / V values.  The
    // appended token (slot ntail - 1 when this call appends it) comes from
    // k_new / v_new.  Every load is issued before the first use (one
    // memory round trip).  All 32 slots lie inside the tail buffer; tokens
    // >= ntail are zeroed after loading, so stale slot contents never reach
    // the MFMAs.
    const _Float16* tk = p.tail_k + toff;
    const _Float16* tv = p.tail_v + toff;
    const int newslot = (fused && seq == total) ? ntail - 1 : -1;
    half8 ka[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int t = 16 * tb + n;
        const _Float16* row = t == newslot ? p.k_new + noff : tk + (size_t)t * kHeadDim;
        ka[kb][tb] = *reinterpret_cast<const half8*>(row + 32 * kb + 8 * w);
      }
    _Float16 va[8][8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = 4 * w + (j >> 1) + 16 * (j & 1);  // tau(w, j)
        const _Float16* row = t == newslot ? p.v_new + noff : tv + (size_t)t * kHeadDim;
        va[mb][j] = row[16 * mb + n];
      }
    floatx4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const half8 z = {};
        acc[tb] = mfma(bq_plain[kb], 16 * tb + n < ntail ? ka[kb][tb] : z, acc[tb]);
      }
    float s0 = n < ntail ? acc[0][0] : -INFINITY;
    float s1 = 16 + n < ntail ? acc[1][0] : -INFINITY;
    softmax_step(st, s0, s1, sl2, n);
    store_p_limbs(sm.pl, w, n, p_limbs(s0, s1));
    wave_lds_sync();
    const half8 z = {};
    const half8 bp = n < 8 ? *reinterpret_cast<const half8*>(&sm.pl[limb][h][pk]) : z;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      half8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = 4 * w + (j >> 1) + 16 * (j & 1);
        a[j] = t < ntail ? va[mb][j] : (_Float16)0.0f;
      }
      st.o[mb] = mfma(a, bp, st.o[mb]);
    }
  }

  // The loop runs two pages per trip so that each ring slot, and with it
  // every LDS address of the page, is a compile-time offset.
  auto page_step = [&](int i, auto slot_c) KITTY_INLINE {
    constexpr int slot = decltype(slot_c)::value;
    wait_page<NHI, BITS>(min(kRing - 1, npg - 1 - i));
    attend_page(sm.ring[slot], valid_of(i), kPageTokens);
    if (i + kRing < npg) {  // refill this slot
      wait_lgkm0();
      compiler_fence();
      dma_record<NHI, BITS>(rec_of(phys_of(i + kRing)), sm.ring[slot], lane);
    }
  };
  static_assert(kRing == 2, "the page loop alternates two ring slots");
  for (int i = 0; i < npg; i += 2) {
    page_step(i, std::integral_constant<int, 0>{});
    if (i + 1 < npg) page_step(i + 1, std::integral_constant<int, 1>{});
  }

  // ---- the tail wave: the last attended page (sealed by this call, or cut by the bound) -------
  if (tail_wave && extra_page) {
    if (new_page) {
      if (seal_rec != nullptr) {  // read the record back through the device coherence point
        wait_lgkm0();  // the quantizer's LDS reads are done before the ring is refilled
        compiler_fence();
        wait_vmcnt<0>();  // the record's stores are complete
        compiler_fence();
        dma_record<NHI, BITS, 16>(seal_rec, sm.ring[0], lane);
        wait_page<NHI, BITS>(0);
        attend_page(sm.ring[0], true, last_lim);
        wave_lds_sync();
      }
    } else {
      const int phys = p.block_table[page_row + P - 1];  // wave-uniform
      if (phys >= 0 && phys < np32) {
        wait_lgkm0();  // the loop's LDS reads are done before the ring is refilled
        compiler_fence();
        dma_record<NHI, BITS>(rec_of(phys), sm.ring[0], lane);
        wait_page<NHI, BITS>(0);
        attend_page(sm.ring[0], true, last_lim);
        wave_lds_sync();
      }
    }
  }

  // ---- this wave's partial (m, l, O with corrections) into its LDS area --------
  const float l_row = row_sum16(st.l);  // head w's denominator over this wave's tokens
  const float m_h = head_of_column(st.m, n), l_h = head_of_column(l_row, n);
  // correction MFMA: rows g (vmin . p), columns 8 + h (hi limb of p) and
  // 12 + h (lo limb); lanes 12..15 of row group 0 add column n - 4.
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float v = st.corr[i4] + dpp<kRowRor4>(st.corr[i4]);
    if (n >= 12 && w == 0) sm.red[n - 12][i4] = v;
  }
  wave_lds_sync();
  // The DPP sums run with every lane active (a DPP read of an inactive lane
  // returns 0); only the stores are predicated.
  floatx4 ov[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int g = mb >> 1;
    const float cg = sm.red[h][g];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) ov[mb][i4] = st.o[mb][i4] + dpp<kRowRor12>(st.o[mb][i4]) + cg;  // hi + lo column
  }
  if (n < 4) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<floatx4*>(&sm.part[h][16 * mb + 4 * w]) = ov[mb];
    if (w == 0) {
      sm.part[h][128] = m_h;
      sm.part[h][129] = l_h;
    }
  }
  __syncthreads();

  // ---- merge the W wave partials ----------------------------------------------
  // Partials combine by log-sum-exp: M = max m_j, weight f_j = 2^(m_j - M),
  // L = sum f_j l_j, O = sum f_j O_j.  Each thread forms one (head, channel)
  // output from the W partials on its own (m and l are broadcast reads), so
  // every LDS read is issued up front and no second barrier is needed.
  const int nthr = 64 * W;
  // The fused step stores the new length once every wave of the sequence
  // has read the old one: each unit, once all its workgroups are past that
  // read, counts itself at the per-sequence counter (one 128-byte line per
  // sequence), and the last unit stores n0 + 1 and clears the counter.  The
  // atomic is issued before the unit's remaining output work, which hides
  // its round trip.
  int* const seq_counter = p.seq_counters + (size_t)b * kSeqCounterStride;
  int seq_old = 0;
  if (fused && threadIdx.x == 0 && p.n_wg == 1)
    seq_old = __hip_atomic_fetch_add(seq_counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto sequence_arrival = [&](int old, int units) {
    if (fused && threadIdx.x == 0 && old == units - 1) {
      __hip_atomic_store(p.seq_lens + b, n0 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(seq_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto out_of = [&](int o) { return p.out + ((size_t)b * p.n_q_heads + hq0 + (o >> 7)) * kHeadDim + (o & 127); };
  float* gpart = p.partial + ((size_t)b * p.n_q_heads + hq0) * p.n_wg * kPartialStride;
  auto st_ag = [](float* a, float v) { __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto ld_ag = [](const float* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  for (int o = threadIdx.x; o < 4 * kHeadDim; o += nthr) {
    const int hh = o >> 7, ch = o & 127;
    if (hh >= gcount) continue;
    float mj[kMaxWgWaves], lj[kMaxWgWaves], oj[kMaxWgWaves];
    float M = kNegBig;
#pragma unroll
    for (int j = 0; j < kMaxWgWaves; ++j) {
      mj[j] = j < W ? all[j].part[hh][128] : kNegBig;
      lj[j] = j < W ? all[j].part[hh][129] : 0.0f;
      oj[j] = j < W ? all[j].part[hh][ch] : 0.0f;
      M = fmaxf(M, mj[j]);
    }
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxWgWaves; ++j) {
      const float f = __builtin_amdgcn_exp2f(mj[j] - M);
      L += f * lj[j];
      O += f * oj[j];
    }
    if (p.n_wg == 1) {
      *out_of(o) = L > 0.0f ? O / L : 0.0f;
    } else {
      // Partials are agent-scope atomic stores (written through to the device
      // coherence point) and the merging workgroup reads them with agent-scope
      // atomic loads, so no L2 write-back / invalidate is needed anywhere.
      float* d = gpart + ((size_t)hh * p.n_wg + blockIdx.x) * kPartialStride;
      st_ag(d + 2 + ch, O);
      if (ch == 0) {
        st_ag(d, M);
        st_ag(d + 1, L);
      }
    }
  }
  if (p.n_wg == 1) {
    sequence_arrival(seq_old, p.n_kv_heads * p.n_head_groups);
    return;
  }

  // ---- several workgroups: count arrivals, the last one merges ---------------------
  compiler_fence();
  wait_vmcnt<0>();  // this thread's partial stores are complete before the workgroup arrives
  compiler_fence();
  __syncthreads();
  int* counter = p.counters + ((size_t)b * p.n_kv_heads + hk) * p.n_head_groups + hg;
  if (threadIdx.x == 0) all[0].flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (all[0].flag != p.n_wg - 1) return;
  compiler_fence();
  if (fused && threadIdx.x == 0)  // the unit is complete: count it for the sequence
    seq_old = __hip_atomic_fetch_add(seq_counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int o = threadIdx.x; o < 4 * kHeadDim; o += nthr) {
    const int hh = o >> 7, ch = o & 127;
    if (hh >= gcount) continue;
    const float* src = gpart + (size_t)hh * p.n_wg * kPartialStride;
    float M = kNegBig, L = 0.0f, O = 0.0f;
    for (int k0 = 0; k0 < p.n_wg; k0 += 4) {  // four partials per round trip, folded online
      float ms[4], ls[4], os[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // every load issued before the first use
        const float* sk = src + min(k0 + k, p.n_wg - 1) * kPartialStride;  // in bounds; masked below
        ms[k] = ld_ag(sk);
        ls[k] = ld_ag(sk + 1);
        os[k] = ld_ag(sk + 2 + ch);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k0 + k >= p.n_wg) {
          ms[k] = kNegBig;
          ls[k] = 0.0f;
          os[k] = 0.0f;
        }
      const float Mn = fmaxf(fmaxf(M, fmaxf(ms[0], ms[1])), fmaxf(ms[2], ms[3]));
      const float a = __builtin_amdgcn_exp2f(M - Mn);
      L *= a;
      O *= a;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float f = __builtin_amdgcn_exp2f(ms[k] - Mn);
        L += f * ls[k];
        O += f * os[k];
      }
      M = Mn;
    }
    *out_of(o) = L > 0.0f ? O / L : 0.0f;
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  sequence_arrival(seq_old, p.n_kv_heads * p.n_head_groups);
}

template <int NHI, int BITS, bool RUN>
hipError_t launch_decode_nbr(const DecodeParams& p, hipStream_t stream) {
  constexpr int wmax = max_wg_waves<NHI, BITS>();
  if (p.wg_waves < 2 || p.wg_waves > wmax) return hipErrorInvalidValue;
  const size_t lds = sizeof(Lds<NHI, BITS>) * p.wg_waves + kZeroRowBytes;
  static const hipError_t attr =  // once per instantiation: allow the largest workgroup's LDS
      hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<NHI, BITS, RUN>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)(sizeof(Lds<NHI, BITS>) * wmax + kZeroRowBytes));
  if (attr != hipSuccess) return attr;
  dim3 grid(p.n_wg, p.n_kv_heads * p.n_head_groups, p.batch);
  hipLaunchKernelGGL((decode_kernel<NHI, BITS, RUN>), grid, dim3(64 * p.wg_waves), lds, stream, p);
  return hipGetLastError();
}

template <int NHI, int BITS>
hipError_t launch_decode_nb(const DecodeParams& p, hipStream_t stream) {
  // only the fused step uses the running sums; plain decode attention reads records alone
  if (p.k_new && p.key_stats) return launch_decode_nbr<NHI, BITS, true>(p, stream);
  return launch_decode_nbr<NHI, BITS, false>(p, stream);
}

template <int NHI>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  if (p.lo_bit == 4) return launch_decode_nb<NHI, 4>(p, stream);
  if (p.lo_bit == 2) return launch_decode_nb<NHI, 2>(p, stream);
  return hipErrorInvalidValue;
}

template <int NHI>
int max_wg_waves_t(int lo_bit) {
  return lo_bit == 4 ? max_wg_waves<NHI, 4>() : max_wg_waves<NHI, 2>();
}

}  // namespace

// Largest page range any page wave gets under plan (n_wg, W) for Pm pages
// (the same weighted division the kernel computes).
static long max_range(long Pm, long n_wg, long W) {
  const long tw = tail_weight((int)W);
  const long wsum = n_wg * weight_prefix(W, W) - page_weight(W - 1) + tw;
  long best = 0;
  for (long pw = 0; pw < n_wg * W; ++pw) {
    const long c0 = (pw / W) * weight_prefix(W, W) + weight_prefix(pw % W, W);
    const long wt = pw == n_wg * W - 1 ? tw : page_weight(pw % W);
    const long r = ((c0 + wt) * Pm) / wsum - (c0 * Pm) / wsum;
    if (r > best) best = r;
  }
  return best;
}

int decode_max_wg_waves(int n_hi, int lo_bit) {
  switch (boost_slots(n_hi)) {
    case 0: return max_wg_waves_t<0>(lo_bit);
    case 16: return max_wg_waves_t<16>(lo_bit);
    case 32: return max_wg_waves_t<32>(lo_bit);
    case 48: return max_wg_waves_t<48>(lo_bit);
    case 64: return max_wg_waves_t<64>(lo_bit);
    case 80: return max_wg_waves_t<80>(lo_bit);
    case 96: return max_wg_waves_t<96>(lo_bit);
    case 112: return max_wg_waves_t<112>(lo_bit);
    case 128: return max_wg_waves_t<128>(lo_bit);
    default: return kMaxWgWaves;
  }
}

// Workgroups of this kernel that one CU holds at once.  Registers allow 3
// waves per SIMD, and the waves of a workgroup go to the CU's 4 SIMDs in
// turn: workgroups of up to 4 waves pack until every SIMD holds 3 (12 / W of
// them), but a second workgroup of 5 to 11 waves finds one of its SIMDs full
// and waits for another CU (measured with a residency probe: 6, 4 and 3
// workgroups of 2, 3 and 4 waves share a CU, workgroups of 5, 6, 8 or 12
// waves run alone).  LDS may allow fewer.
static long wgs_per_cu(long W, int wmax) {
  const long by_simd = W <= 4 ? 12 / W : 1;
  const long by_lds = wmax / W;  // wmax waves' LDS fit one CU
  return by_lds < 1 ? 1 : (by_simd < by_lds ? by_simd : by_lds);
}

// A single-workgroup plan that needs more workgroups than there are CUs, with
// a workgroup size that runs alone on a CU, leaves SIMD slots idle: take
// instead the size among 2, 3, 4 and wmax waves that needs the fewest rounds
// of resident workgroups times (pages per wave + 2), the 2 standing for a
// round's start and merge.  Only the workgroup size changes, so the workspace
// (sized by n_wg) does not.
static SplitPlan pack_workgroups(SplitPlan plan, long P, long units, int wmax, long cus) {
  if (plan.n_wg != 1 || plan.wg_waves <= 4 || plan.wg_waves >= wmax || units <= cus) return plan;
  auto cost = [&](long W) {
    const long per_round = cus * wgs_per_cu(W, wmax);
    return (units + per_round - 1) / per_round * (max_range(P, 1, W) + 2);
  };
  long best = plan.wg_waves, best_cost = cost(best);
  for (long W : {2L, 3L, 4L, (long)wmax}) {
    if (W > wmax || max_range(P, 1, W) > 64) continue;
    const long c = cost(W);
    if (c < best_cost) {
      best = W;
      best_cost = c;
    }
  }
  plan.wg_waves = (int)best;
  return plan;
}

SplitPlan plan_splits(int batch, int n_kv_heads, int n_head_groups, int max_seq_len, int wmax, int cus) {
  const long P = max_seq_len / kPageTokens;
  const long units = (long)batch * n_kv_heads * n_head_groups;
  const long resident = (long)wmax * cus;  // waves: up to 3 per SIMD on every CU, as LDS allows
  long wpu = resident / units;         // waves per unit, the tail wave included
  if (wpu > P + 1) wpu = P + 1;        // at least one page per page wave
  if (wpu < 2) wpu = 2;
  // Every quantity below is non-decreasing in max_seq_len, so a workspace
  // sized for a bound serves every shorter call.
  for (;;) {
    long n_wg = (wpu + wmax - 1) / wmax;
    if (n_wg > kMaxWg) n_wg = kMaxWg;
    long wg_waves = (wpu + n_wg - 1) / n_wg;
    if (wg_waves > wmax) wg_waves = wmax;
    // a page wave keeps its page ids in one 64-lane register; wpu only
    // grows, and for every supported length (P <= 4096) it stops well
    // before 16 x 12 waves
    if (max_range(P, n_wg, wg_waves) <= 64 || n_wg * wg_waves >= (long)kMaxWg * wmax)
      return pack_workgroups(SplitPlan{(int)n_wg, (int)wg_waves}, P, units, wmax, cus);
    ++wpu;
  }
}

// Fills n 32-bit words with zero (a kernel rather than hipMemsetAsync, so
// that a caller may capture it in a HIP graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  switch (boost_slots(p.n_hi)) {  // instantiations by boost slots; the seal ranks p.n_hi channels
    case 0: return launch_decode_t<0>(p, stream);
    case 16: return launch_decode_t<16>(p, stream);
    case 32: return launch_decode_t<32>(p, stream);
    case 48: return launch_decode_t<48>(p, stream);
    case 64: return launch_decode_t<64>(p, stream);
    case 80: return launch_decode_t<80>(p, stream);
    case 96: return launch_decode_t<96>(p, stream);
    case 112: return launch_decode_t<112>(p, stream);
    case 128: return launch_decode_t<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kitty
