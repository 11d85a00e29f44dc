/*
 * kitty_bench.h -- measurement entry points of the Kitty library (gfx950):
 * the HBM read-stream ceiling that the decode kernel's bandwidth is judged
 * against, and the read-and-write stream of the prefill quantizer.  Not
 * part of the cache's hot path; bench.py --ceiling calls them.
 *
 * "Kitty: Accurate and Efficient 2-bit KV Cache Quantization with Dynamic
 * Channel-wise Precision Boost", Abstract: the KV cache is the dominant
 * memory bottleneck of decode, so the rate at which a kernel can read it is
 * the figure of merit, and this is the best rate a read-only kernel reaches.
 */
#ifndef KITTY_BENCH_H
#define KITTY_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every access of these kernels carries the non-temporal cache hint (the
 * data is touched once), as the decode and quantize kernels' streams do. */
enum {
  KITTY_READ_VGPR = 0,        /* 16-byte loads into registers, `depth` in flight per lane, grid-stride */
  KITTY_READ_LDS_RECORDS = 1, /* 3360-byte records streamed into a `depth`-slot LDS ring per wave
                                 with global_load_lds_dwordx4 (the decode kernel's memory path) */
  KITTY_READ_LDS_HEADS = 2    /* the same, in the decode kernel's order: the records form 8
                                 interleaved streams (record 8j + h is page j of head h), and
                                 the sweep takes them one stream after another, so a wave reads
                                 records 8 apart, as a decode wave reads one KV head's pages */
};

/* Read `bytes` of device memory at `src` once (16-byte aligned, a multiple
 * of 16; LDS mode: the whole 3360-byte records it holds) with the access
 * pattern `mode`, on `waves_per_cu` waves per compute unit of the stream's
 * device (VGPR mode: 4..32, a multiple of 4; depth 1, 2, 4 or 8.  LDS modes:
 * one workgroup of 1..12 waves per CU; depth 1..4; waves * depth * 3360
 * bytes of LDS at most 160 KiB).  sink: device uint32 [sink_len], at least
 * one entry per workgroup (VGPR) or per wave (LDS); the kernels keep every
 * load live by storing a checksum there only when it equals a constant, so
 * in practice they write nothing.  Asynchronous on `stream`.  Returns 0,
 * KITTY_ERR_INVALID_ARG (-1) for arguments outside these ranges (before any
 * launch) or KITTY_ERR_HIP (-4). */
int kitty_read_ceiling(const void* src, size_t bytes, int32_t mode, int32_t waves_per_cu, int32_t depth,
                       uint32_t* sink, size_t sink_len, void* stream);

/* The prefill quantizer's memory traffic without its arithmetic, the
 * ceiling its bandwidth is judged against ("Kitty -- Dynamic Channel-wise
 * Mixed-Precision Keys", How it works / Prefill phase: every page of fp16
 * K and V is read once and one packed record is written per page and KV
 * head).  `units` blocks of 128 threads; block u reads `read_bytes` at
 * src + u * read_bytes (thread t XORs the 16-byte words t, t + 128, ...,
 * every load issued before the first use) and writes `write_bytes` at
 * dst + u * write_bytes: 16-byte word j is thread (j mod 128)'s XOR with
 * each of its four 32-bit lanes XORed with j, so every load is live and the
 * writes are real.  src, dst: device memory, 16-byte aligned, not
 * overlapping; read_bytes = 2048 * w for w in {1, 2, 4, 8, 16, 32};
 * write_bytes a multiple of 16 in [2048, 65536] (every thread writes, so
 * every load is needed); 1 <= units < 2^31.
 * Asynchronous on `stream`.  Returns 0, KITTY_ERR_INVALID_ARG (-1) for
 * arguments outside these ranges (before any launch) or KITTY_ERR_HIP (-4). */
int kitty_stream_ceiling(const void* src, void* dst, int64_t units, int32_t read_bytes, int32_t write_bytes,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KITTY_BENCH_H */
