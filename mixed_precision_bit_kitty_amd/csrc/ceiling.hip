// HBM read-stream ceiling (gfx950): kernels that only read memory, the
// reference point for the decode kernel's bandwidth ("Kitty: Accurate and
// Efficient 2-bit KV Cache Quantization with Dynamic Channel-wise Precision
// Boost", Abstract: the KV cache is the dominant memory bottleneck of decode,
// so its read rate is the figure of merit).
//
//  * read_vgpr_kernel: plain 16-byte loads into registers, DEPTH independent
//    loads in flight per lane, a grid-stride sweep over the buffer (each
//    wave instruction reads 1 KiB contiguous);
//  * read_lds_kernel: the decode kernel's memory path without its
//    arithmetic -- each wave streams 3360-byte records (one page record of a
//    KV head at n_hi 32, lo_bit 2) into a DEPTH-slot LDS ring with
//    global_load_lds_dwordx4, waiting for the oldest record before reusing
//    its slot.
//
// Neither writes memory except a per-thread XOR that is stored only when it
// equals a constant (in practice never), which keeps every load live.
// Every access carries the non-temporal hint, as the data is touched once:
// on gfx950 it raises both read-only kernels from 0.77-0.79 to 0.88 of the
// HBM peak (the decode kernel's record DMA and the quantizer use it too).
//
//  * stream_kernel: the prefill quantizer's traffic without its arithmetic
//    (kitty_stream_ceiling) -- one block of two waves per unit reads the
//    unit (a page-head's fp16 K and V: 16 KiB) and writes a record-sized
//    output derived from it, so reads and writes mix as in the quantizer.
#include "kitty_internal.h"
#include "../../include/kitty.h"
#include "../../include/kitty_bench.h"

namespace kitty {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kNever = 0x9E3779B9u;
constexpr int kNt = 2;  // the nt bit of global_load_lds's cache-policy operand
constexpr int kCeilRec = 3360;                  // bytes per record (n_hi 32, lo_bit 2)
constexpr int kCeilSlot = (kCeilRec + 15) / 16 * 16;

template <int DEPTH>
__global__ __launch_bounds__(256) void read_vgpr_kernel(const u32x4* __restrict__ src, size_t n16, uint32_t* sink) {
  const size_t nthr = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (DEPTH - 1) * nthr < n16; i += DEPTH * nthr) {
    u32x4 v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) v[d] = __builtin_nontemporal_load(&src[i + d * nthr]);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= v[d];
  }
  for (; i < n16; i += nthr) acc ^= __builtin_nontemporal_load(&src[i]);
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kNever) sink[blockIdx.x] = x;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One record into an LDS slot: three 1 KiB instructions and one of 288 bytes
// (lanes 0..17), four vector memory instructions in all.
__device__ __forceinline__ void dma_rec(const uint8_t* rec, uint8_t* slot, int lane) {
  const uint8_t* s = rec + 16 * lane;
  __builtin_amdgcn_global_load_lds(s, (lds_void*)slot, 16, 0, kNt);
  __builtin_amdgcn_global_load_lds(s, (lds_void*)slot, 16, 1024, kNt);
  __builtin_amdgcn_global_load_lds(s, (lds_void*)slot, 16, 2048, kNt);
  if (16 * lane < kCeilRec - 3072) __builtin_amdgcn_global_load_lds(s, (lds_void*)slot, 16, 3072, kNt);
}

// Wave g of G takes records [g * n / G, (g + 1) * n / G) of the sweep in
// order.  HEADS: sweep record r is record 8 (r mod P) + r / P with P =
// n / 8 (the last n mod 8 records in place), so the sweep takes the 8
// interleaved streams one after another and a wave reads records 8 apart.
template <int DEPTH, bool HEADS>
__global__ __launch_bounds__(64 * 12) void read_lds_kernel(const uint8_t* __restrict__ src, int64_t n_rec,
                                                           uint32_t* sink) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t G = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t g = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  const int64_t r0 = g * n_rec / G, r1 = (g + 1) * n_rec / G;
  uint8_t* ring = lds + (size_t)wave * DEPTH * kCeilSlot;
  const int n = (int)(r1 - r0);
  const int64_t P8 = n_rec / 8;
  auto rec = [&](int64_t r) { return HEADS && r < 8 * P8 ? 8 * (r % P8) + r / P8 : r; };  // in [0, n_rec)
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < n) dma_rec(src + rec(r0 + d) * kCeilRec, ring + d * kCeilSlot, lane);
  uint32_t acc = 0;
  for (int i = 0; i < n; ++i) {
    const int ahead = min(DEPTH - 1, n - 1 - i);  // records issued after record i
    asm volatile("" ::: "memory");
    if (ahead >= DEPTH - 1) wait_vmcnt<4 * (DEPTH - 1)>();
    else if (ahead == 2) wait_vmcnt<8>();
    else if (ahead == 1) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    uint8_t* slot = ring + (i % DEPTH) * kCeilSlot;
    acc ^= *reinterpret_cast<const uint32_t*>(slot + 4 * lane);  // a read of the landed record
    if (i + DEPTH < n) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      dma_rec(src + rec(r0 + i + DEPTH) * kCeilRec, slot, lane);
    }
  }
  if (acc == kNever) sink[blockIdx.x * (blockDim.x >> 6) + wave] = acc;
}

// Block u: thread t XORs words t + 128 i (i < W) of its unit, all loads
// issued first, then writes words j = t, t + 128, ... < nw of the unit's
// output as that XOR ^ j.
template <int W>
__global__ __launch_bounds__(128) void stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int nw) {
  const int64_t u = blockIdx.x;
  const int t = threadIdx.x;
  const u32x4* s = src + u * (128 * W) + t;
  u32x4 v[W];
#pragma unroll
  for (int i = 0; i < W; ++i) v[i] = __builtin_nontemporal_load(&s[128 * i]);
  u32x4 acc = v[0];
#pragma unroll
  for (int i = 1; i < W; ++i) acc ^= v[i];
  u32x4* d = dst + u * nw;
  for (int j = t; j < nw; j += 128) __builtin_nontemporal_store(acc ^ (uint32_t)j, &d[j]);
}

template <int W>
hipError_t launch_stream(const void* src, void* dst, int64_t units, int nw, hipStream_t s) {
  hipLaunchKernelGGL(stream_kernel<W>, dim3((unsigned)units), dim3(128), 0, s, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), nw);
  return hipGetLastError();
}

template <int DEPTH, bool HEADS>
hipError_t launch_lds(const uint8_t* src, int64_t n_rec, int cus, int waves, uint32_t* sink, hipStream_t s) {
  const size_t lds = (size_t)waves * DEPTH * kCeilSlot;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&read_lds_kernel<DEPTH, HEADS>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((read_lds_kernel<DEPTH, HEADS>), dim3(cus), dim3(64 * waves), lds, s, src, n_rec, sink);
  return hipGetLastError();
}
template <bool HEADS>
hipError_t launch_lds_depth(const uint8_t* src, int64_t n_rec, int cus, int waves, int depth, uint32_t* sink,
                            hipStream_t s) {
  switch (depth) {
    case 1: return launch_lds<1, HEADS>(src, n_rec, cus, waves, sink, s);
    case 2: return launch_lds<2, HEADS>(src, n_rec, cus, waves, sink, s);
    case 3: return launch_lds<3, HEADS>(src, n_rec, cus, waves, sink, s);
    default: return launch_lds<4, HEADS>(src, n_rec, cus, waves, sink, s);
  }
}

template <int DEPTH>
hipError_t launch_vgpr(const void* src, size_t bytes, int cus, int waves, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(read_vgpr_kernel<DEPTH>, dim3(cus * waves / 4), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace
}  // namespace kitty

extern "C" int kitty_read_ceiling(const void* src, size_t bytes, int32_t mode, int32_t waves_per_cu, int32_t depth,
                                  uint32_t* sink, size_t sink_len, void* stream) {
  if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 15) || bytes < 16 || bytes % 16) return KITTY_ERR_INVALID_ARG;
  if (mode == KITTY_READ_VGPR) {
    if (waves_per_cu < 4 || waves_per_cu > 32 || waves_per_cu % 4) return KITTY_ERR_INVALID_ARG;
    if (depth != 1 && depth != 2 && depth != 4 && depth != 8) return KITTY_ERR_INVALID_ARG;
  } else if (mode == KITTY_READ_LDS_RECORDS || mode == KITTY_READ_LDS_HEADS) {
    if (waves_per_cu < 1 || waves_per_cu > 12 || depth < 1 || depth > 4) return KITTY_ERR_INVALID_ARG;
    if ((size_t)waves_per_cu * depth * kitty::kCeilSlot > 160 * 1024) return KITTY_ERR_INVALID_ARG;
    if (bytes < (size_t)kitty::kCeilRec) return KITTY_ERR_INVALID_ARG;
  } else {
    return KITTY_ERR_INVALID_ARG;
  }
  int dev = 0, cus = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamGetDevice(s, &dev) != hipSuccess && hipGetDevice(&dev) != hipSuccess) return KITTY_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return KITTY_ERR_HIP;
  (void)hipGetLastError();
  hipError_t e;
  if (mode == KITTY_READ_VGPR) {
    if (sink_len < (size_t)cus * waves_per_cu / 4) return KITTY_ERR_INVALID_ARG;
    switch (depth) {
      case 1: e = kitty::launch_vgpr<1>(src, bytes, cus, waves_per_cu, sink, s); break;
      case 2: e = kitty::launch_vgpr<2>(src, bytes, cus, waves_per_cu, sink, s); break;
      case 4: e = kitty::launch_vgpr<4>(src, bytes, cus, waves_per_cu, sink, s); break;
      default: e = kitty::launch_vgpr<8>(src, bytes, cus, waves_per_cu, sink, s); break;
    }
  } else {
    if (sink_len < (size_t)cus * waves_per_cu) return KITTY_ERR_INVALID_ARG;
    const int64_t n_rec = (int64_t)(bytes / kitty::kCeilRec);
    const uint8_t* p = static_cast<const uint8_t*>(src);
    e = mode == KITTY_READ_LDS_HEADS ? kitty::launch_lds_depth<true>(p, n_rec, cus, waves_per_cu, depth, sink, s)
                                     : kitty::launch_lds_depth<false>(p, n_rec, cus, waves_per_cu, depth, sink, s);
  }
  return e == hipSuccess ? KITTY_OK : KITTY_ERR_HIP;
}

extern "C" int kitty_stream_ceiling(const void* src, void* dst, int64_t units, int32_t read_bytes, int32_t write_bytes,
                                    void* stream) {
  if (!src || !dst || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
    return KITTY_ERR_INVALID_ARG;
  if (units < 1 || units > 0x7FFFFFFF) return KITTY_ERR_INVALID_ARG;
  const int w = read_bytes / 2048;
  if (read_bytes % 2048 || (w != 1 && w != 2 && w != 4 && w != 8 && w != 16 && w != 32)) return KITTY_ERR_INVALID_ARG;
  if (write_bytes < 2048 || write_bytes > 65536 || write_bytes % 16) return KITTY_ERR_INVALID_ARG;  // >= 128 words
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t rs = (uintptr_t)units * (uintptr_t)read_bytes, ws = (uintptr_t)units * (uintptr_t)write_bytes;
  if (s0 > UINTPTR_MAX - rs || d0 > UINTPTR_MAX - ws) return KITTY_ERR_INVALID_ARG;  // ranges wrap the address space
  if (s0 < d0 + ws && d0 < s0 + rs) return KITTY_ERR_INVALID_ARG;                     // overlapping
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int nw = write_bytes / 16;
  hipError_t e;
  switch (w) {
    case 1: e = kitty::launch_stream<1>(src, dst, units, nw, s); break;
    case 2: e = kitty::launch_stream<2>(src, dst, units, nw, s); break;
    case 4: e = kitty::launch_stream<4>(src, dst, units, nw, s); break;
    case 8: e = kitty::launch_stream<8>(src, dst, units, nw, s); break;
    case 16: e = kitty::launch_stream<16>(src, dst, units, nw, s); break;
    default: e = kitty::launch_stream<32>(src, dst, units, nw, s); break;
  }
  return e == hipSuccess ? KITTY_OK : KITTY_ERR_HIP;
}
