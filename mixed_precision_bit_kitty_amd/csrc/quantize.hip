// Prefill and append/seal kernels for gfx950.  One wave quantizes one
// (page of 32 tokens, KV head) with quantize_page_wave (page_quant.h): Key
// channel statistics and the Dynamic Channel-wise Precision Boost ranking
// ("Kitty: Accurate and Efficient 2-bit KV Cache Quantization with Dynamic
// Channel-wise Precision Boost", Abstract; "Kitty -- Dynamic Channel-wise
// Mixed-Precision Keys", How it works / Prefill phase, steps 1-3), two-plane
// Key codes and lo_bit Value codes.  In the running ranking mode the
// boosted channels come from the head's exact running sums instead
// (key_chunk_kernel, key_rank_kernel and the append below).
#include "kitty_internal.h"
#include "page_quant.h"

#pragma clang fp contract(off)

namespace kitty {
namespace {

using namespace pq;

typedef __attribute__((address_space(3))) void lds_void;

// Copy the 8 KB of a page's values (32 contiguous rows) into LDS with the
// LDS DMA path, 1 KB per instruction, non-temporal (nt: the inputs are read
// once); returns once they have landed.
constexpr int kNt = 2;  // the nt bit of the cache-policy operand
__device__ __forceinline__ void stage_value_page(const _Float16* src, uint8_t* dst, int lane) {
  const uint8_t* s0 = reinterpret_cast<const uint8_t*>(src) + 16 * lane;
  const uint8_t* s1 = s0 + 4096;
  __builtin_amdgcn_global_load_lds(s0, (lds_void*)dst, 16, 0, kNt);
  __builtin_amdgcn_global_load_lds(s0, (lds_void*)dst, 16, 1024, kNt);
  __builtin_amdgcn_global_load_lds(s0, (lds_void*)dst, 16, 2048, kNt);
  __builtin_amdgcn_global_load_lds(s0, (lds_void*)dst, 16, 3072, kNt);
  __builtin_amdgcn_global_load_lds(s1, (lds_void*)(dst + 4096), 16, 0, kNt);
  __builtin_amdgcn_global_load_lds(s1, (lds_void*)(dst + 4096), 16, 1024, kNt);
  __builtin_amdgcn_global_load_lds(s1, (lds_void*)(dst + 4096), 16, 2048, kNt);
  __builtin_amdgcn_global_load_lds(s1, (lds_void*)(dst + 4096), 16, 3072, kNt);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int mask) {
  const uint32_t lo = __shfl_xor((uint32_t)x, mask), hi = __shfl_xor((uint32_t)(x >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}

// Running ranking mode, ahead of the prefill ("Kitty -- Dynamic
// Channel-wise Mixed-Precision Keys", How it works / Prefill phase, steps 1
// and 5): the exact running sums of every filled (sequence, KV head) over
// its n_b tokens (tail included) become its state, and their ranking is
// stored for quantize_pages_kernel.  Integer sums may be added in any
// order, so the work is split in chunks of kChunkPages pages:
//  * key_chunk_kernel sums one chunk and writes the partial sums into the
//    record slot of the chunk's first page, which quantize_pages_kernel
//    overwrites later (3072 bytes; every record is at least that long);
//  * key_rank_kernel adds the partials of a (sequence, KV head) and the
//    tokens of a chunk without a sealed page (fewer than 32 tail tokens),
//    stores the state and ranks it.
constexpr int kChunkPages = 8;
constexpr int kChunkTokens = kChunkPages * kPageTokens;
static_assert(rec_bytes(0, 2) >= kStatsCopy, "a chunk's partial sums fit the smallest record");

__device__ __forceinline__ int prefill_len(const QuantizeParams& p, int b) {
  const int n = p.lens ? p.lens[b] : p.S;
  return n > p.S ? p.S : n;  // negative: the sequence is left as it is
}
// the record slot of (b, page, h), or null when its block table entry is invalid
__device__ __forceinline__ uint8_t* record_of(const QuantizeParams& p, int b, int page, int h) {
  const int phys = p.block_table[(size_t)b * p.max_pages + page];
  if (phys < 0 || (int64_t)phys >= p.n_pages) return nullptr;
  return p.pages + (int64_t)phys * p.page_bytes + (int64_t)h * rec_bytes(boost_slots(p.n_hi), p.lo_bit);
}

// Chunk sums in float64, exactly.  For a = k 2^24 (the fixed-point value of
// one fp16 key, as in accumulate: an integer, |a| < 2^40) split as a = h 2^20
// + l with h = trunc(a / 2^20) and |h|, |l| < 2^20 (both with a's sign):
// a^2 = h^2 2^40 + 2 h l 2^20 + l^2.  The sums are kept in units that need
// no per-key scaling: k itself (a = k 2^24), h = trunc(16 k) and
// r = k - h / 16 (l = r 2^24), so that the float64 values are sum k (a
// multiple of 2^-24), sum h^2 (an integer), sum h r (a multiple of 2^-24)
// and sum r^2 (a multiple of 2^-48).  Over a lane's 32 terms each stays
// below 2^45 of its unit, so every float64 add and FMA is exact, and
// scaling by 2^24, 2^24 and 2^48 at the end gives the integers sum a,
// sum h l and sum l^2 (float64 runs at the float32 vector rate on this
// part, and the integer form took 64-bit shifts, masks and carries per
// term).
struct ChunkSums {
  double s1;  // sum k
  double hh;  // sum h^2
  double hl;  // sum h r (>= 0: h and r share k's sign)
  double ll;  // sum r^2
};
__device__ __forceinline__ void chunk_add(uint32_t h16, ChunkSums& c) {
  const double k = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)h16);  // exact
  c.s1 += k;
  const double h = __builtin_trunc(k * 16.0);
  const double r = __builtin_fma(h, -0.0625, k);
  c.hh = __builtin_fma(h, h, c.hh);
  c.hl = __builtin_fma(h, r, c.hl);
  c.ll = __builtin_fma(r, r, c.ll);
}
// an integral float64 of magnitude below 2^53 as int64, exactly
__device__ __forceinline__ int64_t exact_i64(double x) {
  const double hi = __builtin_floor(x * 0x1p-32);
  const double lo = __builtin_fma(hi, -4294967296.0, x);  // in [0, 2^32)
  return (int64_t)(((uint64_t)(uint32_t)(int32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// grid (chunks, Hkv, batch), 4 waves.  Lane (cb = lane & 31, tg = lane >> 5)
// of wave w sums channels 4cb .. 4cb + 3 over tokens 32j + tg + 2i (i =
// 0..15) of pages j = 8c + 2w, 8c + 2w + 1 of chunk c (four channels a lane
// keep the accumulators within four waves per SIMD).
__global__ __launch_bounds__(256) void key_chunk_kernel(QuantizeParams p) {
  __shared__ int64_t ws1[4][kHeadDim];
  __shared__ u128 ws2[4][kHeadDim];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, cb = lane & 31, tg = lane >> 5;
  const int n = prefill_len(p, b);
  const int P = n < 0 ? 0 : n / kPageTokens;
  if (kChunkPages * chunk >= P) return;  // no sealed page here: key_rank_kernel sums these tokens (block-uniform)
  const int t_end = min(n, kChunkTokens * (chunk + 1));
  const _Float16* kb = p.k + ((size_t)b * p.n_kv_heads + h) * (size_t)p.S * kHeadDim + 4 * cb;
  ChunkSums acc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = ChunkSums{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int pg = 0; pg < 2; ++pg) {
    const int t0 = kChunkTokens * chunk + kPageTokens * (2 * wave + pg);
    u32x2 rows[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // every load issued before the first use
      const int t = t0 + tg + 2 * i;
      rows[i] = t < t_end ? *reinterpret_cast<const u32x2*>(kb + (size_t)t * kHeadDim) : u32x2{0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)  // +0 halves of skipped tokens add nothing
        chunk_add((rows[i][e >> 1] >> (16 * (e & 1))) & 0xFFFFu, acc[e]);
  }
  int64_t s1[4];
  u128 s2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s1[e] = exact_i64(acc[e].s1 * 0x1p24);
    s2[e] = ((u128)(uint64_t)exact_i64(acc[e].hh) << 40) + ((u128)(uint64_t)exact_i64(acc[e].hl * 0x1p24) << 21) +
            (u128)(uint64_t)exact_i64(acc[e].ll * 0x1p48);
    s1[e] += (int64_t)shfl_xor_u64((uint64_t)s1[e], 32);  // the other token group
    const uint64_t lo = shfl_xor_u64((uint64_t)s2[e], 32), hi = shfl_xor_u64((uint64_t)(s2[e] >> 64), 32);
    s2[e] += ((u128)hi << 64) | lo;
  }
  if (tg == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ws1[wave][4 * cb + e] = s1[e];
      ws2[wave][4 * cb + e] = s2[e];
    }
  }
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    const int c = threadIdx.x;
    int64_t t1 = ws1[0][c] + ws1[1][c] + ws1[2][c] + ws1[3][c];
    const u128 t2 = ws2[0][c] + ws2[1][c] + ws2[2][c] + ws2[3][c];
    uint8_t* rec = record_of(p, b, kChunkPages * chunk, h);
    if (rec) {
      reinterpret_cast<int64_t*>(rec + kStatsS1)[c] = t1;
      reinterpret_cast<uint64_t*>(rec + kStatsS2Lo)[c] = (uint64_t)t2;
      reinterpret_cast<uint64_t*>(rec + kStatsS2Hi)[c] = (uint64_t)(t2 >> 64);
    }
  }
}

// grid (Hkv, batch), 8 waves: thread (part, c) adds channel c's partials
// of every kRankParts-th run of kRound chunks (part 0 also the tokens of a
// chunk without a sealed page); the parts' totals meet in LDS, wave 0
// stores the state, ranks it and stores the mask.
constexpr int kRankParts = 4;
__global__ __launch_bounds__(kHeadDim * kRankParts) void key_rank_kernel(QuantizeParams p) {
  __shared__ int64_t ts1[kRankParts][kHeadDim];
  __shared__ u128 ts2[kRankParts][kHeadDim];
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x % kHeadDim, part = threadIdx.x / kHeadDim;
  const int lane = threadIdx.x & 63;
  const int n = prefill_len(p, b);
  if (n < 0) return;  // block-uniform
  const int P = n / kPageTokens;
  int64_t s1 = 0;
  u128 s2 = 0;
  const int chunks = (P + kChunkPages - 1) / kChunkPages;  // chunks with a sealed page
  constexpr int kRound = 16;  // chunks per round trip (4096 tokens)
  for (int j0 = part * kRound; j0 < chunks; j0 += kRankParts * kRound) {
    const uint8_t* recs[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) recs[u] = j0 + u < chunks ? record_of(p, b, kChunkPages * (j0 + u), h) : nullptr;
    int64_t v1[kRound];
    uint64_t vlo[kRound], vhi[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) {  // an invalid block table entry: the result is undefined, nothing is read
      v1[u] = recs[u] ? reinterpret_cast<const int64_t*>(recs[u] + kStatsS1)[c] : 0;
      vlo[u] = recs[u] ? reinterpret_cast<const uint64_t*>(recs[u] + kStatsS2Lo)[c] : 0;
      vhi[u] = recs[u] ? reinterpret_cast<const uint64_t*>(recs[u] + kStatsS2Hi)[c] : 0;
    }
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      s1 += v1[u];
      s2 += ((u128)vhi[u] << 64) | vlo[u];
    }
  }
  if (part == 0) {
    const _Float16* kb = p.k + ((size_t)b * p.n_kv_heads + h) * (size_t)p.S * kHeadDim + c;
    for (int t = kChunkTokens * chunks; t < n; ++t)  // fewer than 32 tail tokens
      accumulate(__builtin_bit_cast(uint16_t, kb[(size_t)t * kHeadDim]), s1, s2);
  }
  ts1[part][c] = s1;
  ts2[part][c] = s2;
  __syncthreads();
  uint8_t* st = p.key_stats + ((size_t)b * p.n_kv_heads + h) * kStatsBytes;
  if (threadIdx.x < 64) {
    LaneSums r;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      r.s1[e] = 0;
      r.s2[e] = 0;
#pragma unroll
      for (int q = 0; q < kRankParts; ++q) {
        r.s1[e] += ts1[q][2 * lane + e];
        r.s2[e] += ts2[q][2 * lane + e];
      }
    }
    store_sums(sums_copy(st, (uint32_t)n), lane, r);
    const RankIn rk = running_rank(r, (uint32_t)n, p.n_hi, lane);
    // mask word m: channel 32m + 2i + j at bit 2i + j, from lanes 16m + i
    const uint64_t B0 = __ballot(rk.h0), B1 = __ballot(rk.h1);
    if (lane < 4) {
      auto spread = [](uint32_t x) {  // bit i -> bit 2i, 16 bits
        x = (x | (x << 8)) & 0x00FF00FFu;
        x = (x | (x << 4)) & 0x0F0F0F0Fu;
        x = (x | (x << 2)) & 0x33333333u;
        return (x | (x << 1)) & 0x55555555u;
      };
      const uint32_t w0 = (uint32_t)(B0 >> (16 * lane)) & 0xFFFFu, w1 = (uint32_t)(B1 >> (16 * lane)) & 0xFFFFu;
      reinterpret_cast<uint32_t*>(st + kStatsMask)[lane] = spread(w0) | (spread(w1) << 1);
    }
  }
}

// grid (pages + 1, Hkv, batch), two waves per block: wave 0 quantizes the
// page's keys, wave 1 its values (disjoint parts of one LDS area), so the
// two halves' memory latency overlaps.  The value wave first stages its
// page in LDS, so the per-token steps and the per-channel codes read it
// from there rather than from global memory twice.
template <int NHI, int BITS>
__global__ __launch_bounds__(128) void quantize_pages_kernel(QuantizeParams p) {
  constexpr int kVStage = quant_lds_bytes(NHI);  // the value page: 32 x 128 fp16
  __shared__ __attribute__((aligned(16))) uint8_t lds[kVStage + kPageTokens * kHeadDim * 2];
  const int page = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int n = p.lens ? p.lens[b] : p.S;
  if (n < 0) return;  // a negative length leaves sequence b as it is
  n = n > p.S ? p.S : n;
  int P = n / kPageTokens;
  if (P > p.max_pages) P = p.max_pages;
  const size_t seq_off = ((size_t)b * p.n_kv_heads + h) * (size_t)p.S * kHeadDim;
  if (page < P) {
    const int phys = p.block_table[(size_t)b * p.max_pages + page];
    if (phys < 0 || (int64_t)phys >= p.n_pages) return;
    uint8_t* rec = p.pages + (int64_t)phys * p.page_bytes + (int64_t)h * rec_bytes(NHI, BITS);
    const size_t row0 = seq_off + (size_t)page * kPageTokens * kHeadDim;
    if (wave == 0) {
      // the running mode takes the ranking key_stats_kernel stored (two
      // inlined copies: one register allocation each)
      if (p.key_stats)
        quantize_keys_wave<NHI, BITS>(RowSrc{p.k + row0, nullptr}, rec, lds, p.n_hi,
                                      rank_from_mask(p.key_stats + ((size_t)b * p.n_kv_heads + h) * kStatsBytes, lane));
      else
        quantize_keys_wave<NHI, BITS>(RowSrc{p.k + row0, nullptr}, rec, lds, p.n_hi);
    } else {
      stage_value_page(p.v + row0, lds + kVStage, lane);
      quantize_values_wave<NHI, BITS>(RowSrc{reinterpret_cast<const _Float16*>(lds + kVStage), nullptr}, rec, lds);
    }
  } else if (page == P) {  // the tail: wave 0 copies keys, wave 1 values
    const int nt = n - P * kPageTokens;
    const size_t tail_off = ((size_t)b * p.n_kv_heads + h) * kPageTokens * kHeadDim;
    const _Float16* src_base = wave == 0 ? p.k : p.v;
    _Float16* dst_base = wave == 0 ? p.tail_k : p.tail_v;
    for (int t = 0; t < nt; ++t) {
      const size_t src = seq_off + ((size_t)P * kPageTokens + t) * kHeadDim + 2 * lane;
      const size_t dst = tail_off + (size_t)t * kHeadDim + 2 * lane;
      *reinterpret_cast<uint32_t*>(dst_base + dst) = *reinterpret_cast<const uint32_t*>(src_base + src);
    }
    if (h == 0 && threadIdx.x == 0) p.seq_lens[b] = n;
  }
}

// grid (batch), block = min(Hkv, 8) waves (kWaveLds bytes of LDS each); each wave appends one head at a
// time and seals it when the tail fills; the sequence length is bumped after
// every head of the sequence is done.
template <int NHI, int BITS>
__global__ __launch_bounds__(512) void append_token_kernel(AppendParams p) {  // at most 8 waves
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int n = p.seq_lens[b];
  if (n < 0) return;  // an inactive slot: nothing appended (block-uniform)
  const int slot = n % kPageTokens;
  for (int h = wave; h < p.n_kv_heads; h += nw) {
    const size_t tail_off = ((size_t)b * p.n_kv_heads + h) * kPageTokens * kHeadDim;
    const size_t new_off = ((size_t)b * p.n_kv_heads + h) * kHeadDim;
    const uint32_t k2 = *reinterpret_cast<const uint32_t*>(p.k_new + new_off + 2 * lane);
    *reinterpret_cast<uint32_t*>(p.tail_k + tail_off + (size_t)slot * kHeadDim + 2 * lane) = k2;
    *reinterpret_cast<uint32_t*>(p.tail_v + tail_off + (size_t)slot * kHeadDim + 2 * lane) =
        *reinterpret_cast<const uint32_t*>(p.v_new + new_off + 2 * lane);
    // running mode (Decode phase steps 1-2): the token joins the head's
    // running sums, and a page sealed now is ranked over all n + 1 tokens
    RankIn rk{false, false, false};
    if (p.key_stats) {
      uint8_t* st = p.key_stats + ((size_t)b * p.n_kv_heads + h) * kStatsBytes;
      LaneSums r = load_sums(sums_copy(st, (uint32_t)n), lane);
      add_token(r, k2);
      store_sums(sums_copy(st, (uint32_t)n + 1), lane, r);
      if (slot == kPageTokens - 1) rk = running_rank(r, (uint32_t)n + 1, p.n_hi, lane);
    }
    if (slot == kPageTokens - 1) {
      const int pg = n / kPageTokens;
      if (pg < p.max_pages) {
        const int phys = p.block_table[(size_t)b * p.max_pages + pg];
        if (phys >= 0 && (int64_t)phys < p.n_pages) {
          uint8_t* rec = p.pages + (int64_t)phys * p.page_bytes + (int64_t)h * rec_bytes(NHI, BITS);
          quantize_page_wave<NHI, BITS>(RowSrc{p.tail_k + tail_off, p.k_new + new_off},
                                        RowSrc{p.tail_v + tail_off, p.v_new + new_off}, rec, lds_dyn + wave * kWaveLds,
                                        p.n_hi, rk);
        }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) p.seq_lens[b] = n + 1;
}

template <int NHI>
hipError_t launch_quantize_t(const QuantizeParams& p, hipStream_t stream) {
  if (p.key_stats) {  // running mode: sums and ranking first, on the same stream
    const int chunks = (p.S / kPageTokens + kChunkPages - 1) / kChunkPages;
    if (chunks > 0) hipLaunchKernelGGL(key_chunk_kernel, dim3(chunks, p.n_kv_heads, p.batch), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(key_rank_kernel, dim3(p.n_kv_heads, p.batch), dim3(kHeadDim * kRankParts), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.S / kPageTokens + 1, p.n_kv_heads, p.batch);
  if (p.lo_bit == 4)
    hipLaunchKernelGGL((quantize_pages_kernel<NHI, 4>), grid, dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL((quantize_pages_kernel<NHI, 2>), grid, dim3(128), 0, stream, p);
  return hipGetLastError();
}

template <int NHI>
hipError_t launch_append_t(const AppendParams& p, hipStream_t stream) {
  const int nw = p.n_kv_heads < 8 ? p.n_kv_heads : 8;
  if (p.lo_bit == 4)
    hipLaunchKernelGGL((append_token_kernel<NHI, 4>), dim3(p.batch), dim3(64 * nw), nw * kWaveLds, stream, p);
  else
    hipLaunchKernelGGL((append_token_kernel<NHI, 2>), dim3(p.batch), dim3(64 * nw), nw * kWaveLds, stream, p);
  return hipGetLastError();
}

}  // namespace

// Instantiations by boost slots: n_hi rounded up to a multiple of 16.
#define KITTY_NHI_DISPATCH(fn, nhi, ...)                   \
  switch (boost_slots(nhi)) {                              \
    case 0: return fn<0>(__VA_ARGS__);                     \
    case 16: return fn<16>(__VA_ARGS__);                   \
    case 32: return fn<32>(__VA_ARGS__);                   \
    case 48: return fn<48>(__VA_ARGS__);                   \
    case 64: return fn<64>(__VA_ARGS__);                   \
    case 80: return fn<80>(__VA_ARGS__);                   \
    case 96: return fn<96>(__VA_ARGS__);                   \
    case 112: return fn<112>(__VA_ARGS__);                 \
    case 128: return fn<128>(__VA_ARGS__);                 \
    default: return hipErrorInvalidValue;                  \
  }

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t stream) {
  KITTY_NHI_DISPATCH(launch_quantize_t, p.n_hi, p, stream)
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  KITTY_NHI_DISPATCH(launch_append_t, p.n_hi, p, stream)
}

}  // namespace kitty
