// Internal declarations of the Kitty HIP library (gfx950 only).
//
// Page record of one (page of 32 tokens, KV head) for the default (hi_bit 4,
// lo_bit 2) pair, n = boost slots (n_hi rounded up to a multiple of 16;
// slots n_hi .. n - 1 hold code 0 and index 0) (the two uniform 2-bit Key
// tensors of "Kitty: Accurate and Efficient 2-bit KV Cache Quantization with
// Dynamic Channel-wise Precision Boost", Abstract, plus 2-bit Values and fp16
// metadata):
//
//   0          K base plane    1024 B  64 chunks x 16 B, chunk = one lane's MFMA A operand
//   1024       K boost plane   8n B    one 32-bit word per (lane, 32-slot block)
//   1024+8n    V code plane    1024 B  64 chunks x 16 B
//   2048+8n    kscale          fp16[128]  (4 x step on boosted channels, step elsewhere)
//   2304+8n    kmin            fp16[128]
//   2560+8n    vscale          fp16[4 groups][32], token order kappa
//   2816+8n    vmin            fp16[4][32]
//   3072+8n    idx             uint8[n], ascending boosted channel list
//
// Code word: 16 two-bit codes for two combos A, B of 8 elements e; element e
// of A at bit 16*(e>>2) + 4*(e&1) + 2*((e>>1)&1), of B 8 bits higher.  Byte 0
// holds A's elements 0..3, byte 1 B's, bytes 2 and 3 their elements 4..7,
// and in each byte elements 0, 1 (4, 5) sit in the low two bits of its two
// nibbles, elements 2, 3 (6, 7) in the high two.  With this placement the
// word masked to the nibbles' low bits, and the word shifted right by 2 and
// masked, hold e2m1 nibbles 00cc = c / 2, and eight fp4 conversions (two
// codes each) give both combos' MFMA operands as exact fp16 codes.
//
// Chunk c of a 16-byte plane, u = c & 15, w = c >> 4, word x = 0..3:
//   K base : A = (token u,      channel 32x + 8w + e), B = (token 16 + u, same channel)
//   V codes: A = (token tau(w,e), channel 32x + u),    B = (token tau(w,e), channel 32x + 16 + u)
// tau(w, e) = 4w + (e >> 1) + 16 (e & 1): value index kappa = 8w + e holds
// token kappa / 2 for even kappa and kappa / 2 + 16 for odd kappa, so the two
// tokens t, t + 16 that one lane holds after QK (columns = tokens) are one
// adjacent pair in the P operand of the PV MFMA.
// K boost: nf = n / 32 full slot blocks, word of (chunk c, block b) at byte
// 4*(c*nf + b), slots 32b + 8w + e; if n % 32 == 16 a half block follows at
// byte 256*nf + 4c for chunks c < 32.
//
// The (hi_bit 8, lo_bit 4) pair ("Kitty -- Dynamic Channel-wise
// Mixed-Precision Keys", table "Tuning avg_bits") stores 4-bit planes of the
// same shape: a word holds ONE combo of 8 elements, element e at bit
// 16*(e>>2) + 8*(e&1) + 4*((e>>1)&1), so that each byte holds two codes in
// the low nibbles of the word and of the word shifted right by 4 (e4m3
// bytes 0000cccc = c * 2^-9 for the fp8 conversion); a chunk is 32 B,
// combo A at word 2x and combo B at
// word 2x + 1 (same tokens and channels as above); boost words are pairs at
// byte 8*(c*nf + b) (+4 for B), the half block at 512*nf + 8c.  Sizes: planes
// 2048 B, boost 16n B; metadata as above; 5120 + 17n bytes in total.  In
// general, with b = lo_bit: base 512b, boost 4bn, values 512b, metadata 1024,
// idx n.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kitty {

constexpr int kHeadDim = 128;
constexpr int kPageTokens = 32;
constexpr int kVGroup = 32;

// b = lo_bit (2 or 4); n_hi here is the record's boost slot count, a
// multiple of 16 (boost_slots of the boosted channel count)
__host__ __device__ constexpr int rec_bytes(int n_hi, int b = 2) { return 1024 * b + 4 * b * n_hi + 1024 + n_hi; }
// Boost slots of a record for n_hi boosted channels: n_hi rounded up to a
// multiple of 16; slots n_hi .. boost_slots - 1 hold code 0 and index 0.
__host__ __device__ constexpr int boost_slots(int n_hi) { return (n_hi + 15) / 16 * 16; }
__host__ __device__ constexpr int off_kboost(int b = 2) { return 512 * b; }
__host__ __device__ constexpr int off_v(int n_hi, int b = 2) { return 512 * b + 4 * b * n_hi; }
__host__ __device__ constexpr int off_kscale(int n_hi, int b = 2) { return 1024 * b + 4 * b * n_hi; }
__host__ __device__ constexpr int off_kmin(int n_hi, int b = 2) { return off_kscale(n_hi, b) + 256; }
__host__ __device__ constexpr int off_vscale(int n_hi, int b = 2) { return off_kscale(n_hi, b) + 512; }
__host__ __device__ constexpr int off_vmin(int n_hi, int b = 2) { return off_kscale(n_hi, b) + 768; }
__host__ __device__ constexpr int off_idx(int n_hi, int b = 2) { return off_kscale(n_hi, b) + 1024; }
static_assert(rec_bytes(32) == 3360 && off_idx(32) == 3328 && rec_bytes(32, 4) == 5664, "record layout");

// n_hi: boosted channels (any count 0..128)
__host__ __device__ inline int64_t page_stride_bytes(int n_kv_heads, int n_hi, int b = 2) {
  int64_t raw = (int64_t)n_kv_heads * rec_bytes(boost_slots(n_hi), b);
  return (raw + 255) / 256 * 256;
}

// Launch-side parameters shared by the ABI layer and the kernels.
struct QuantizeParams {
  uint8_t* pages;
  int64_t n_pages;
  int64_t page_bytes;
  const int32_t* block_table;
  int32_t max_pages;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t n_hi;
  int32_t lo_bit;
  _Float16* tail_k;
  _Float16* tail_v;
  int32_t* seq_lens;
  const _Float16* k;
  const _Float16* v;
  int32_t S;
  const int32_t* lens;
  uint8_t* key_stats;      // running ranking mode: [batch][Hkv] states of kKeyStatsBytes; null in the page mode
};

struct AppendParams {
  uint8_t* pages;
  int64_t n_pages;
  int64_t page_bytes;
  const int32_t* block_table;
  int32_t max_pages;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t n_hi;
  int32_t lo_bit;
  _Float16* tail_k;
  _Float16* tail_v;
  int32_t* seq_lens;
  const _Float16* k_new;
  const _Float16* v_new;
  uint8_t* key_stats;      // running ranking mode (see QuantizeParams)
};

struct DecodeParams {
  uint8_t* pages;          // written only by the fused step's seal
  int64_t n_pages;
  int64_t page_bytes;
  const int32_t* block_table;
  int32_t max_pages;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t n_hi;
  int32_t lo_bit;
  _Float16* tail_k;        // written only by the fused step's append
  _Float16* tail_v;
  int32_t* seq_lens;       // written only by the fused step's append
  const _Float16* q;
  const _Float16* k_new;   // fused step: the appended token [batch][Hkv][D]; null for a plain decode
  const _Float16* v_new;
  int32_t n_q_heads;
  int32_t group;           // G = Hq / Hkv
  int32_t n_head_groups;   // ceil(G / 4)
  int32_t max_seq_len;
  int32_t n_wg;            // workgroups per (sequence, KV head, head group)
  int32_t wg_waves;        // waves per workgroup; the unit's last wave also attends over the tail
  float* partial;          // [batch][Hq][n_wg][kPartialStride] per-workgroup partials
  int* counters;           // [batch][Hkv][n_head_groups] workgroup arrival counters, zero between calls
  int* seq_counters;       // [batch] finished units per sequence (fused step), zero between calls
  uint8_t* seal_scratch;   // [batch][Hkv][n_head_groups - 1] records re-quantized by head groups >= 1
  float* out;              // [batch][Hq][D]
  uint8_t* key_stats;      // running ranking mode: the fused step reads copy n & 1 and writes copy (n + 1) & 1
};

constexpr int kPartialStride = 132;  // m, l, O[128], 2 pad floats
constexpr int kMaxWgWaves = 12;      // waves per decode workgroup
constexpr int kMaxWg = 16;           // decode workgroups per (sequence, KV head, head group)
// Longest sequence decode attention accepts: 4096 pages of 32 tokens (+ a
// partial tail page); a wave keeps its page ids in one 64-lane register, and
// 16 workgroups x 9 to 12 waves x 64 pages cover it.
constexpr int kMaxSeqLen = 4096 * 32 + 31;
constexpr int kSeqCounterStride = 32;  // ints: one 128-byte line per sequence counter

// Split-KV plan shared by the workspace query and the launch.
struct SplitPlan {
  int n_wg;
  int wg_waves;
};
// wmax: waves per workgroup that the record size allows (decode_max_wg_waves);
// cus: compute units the launch may use.  Every quantity is non-decreasing in
// max_seq_len and in cus, so a workspace sized for a bound and for
// kMaxCus serves every shorter call on any device with at most kMaxCus CUs.
SplitPlan plan_splits(int batch, int n_kv_heads, int n_head_groups, int max_seq_len, int wmax, int cus);
constexpr int kMaxCus = 256;  // an MI355X (gfx950) has 256 compute units
int decode_max_wg_waves(int n_hi, int lo_bit);

constexpr int kKeyStatsBytes = 8192;  // running-mode state of one (sequence, KV head)
constexpr int kMaxRunningTokens = 1 << 23;  // running mode: exact scores stay below 2^127

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t stream);  // p[0..n) = 0 by a kernel

}  // namespace kitty
