/*
 * kitty.h -- C ABI of the Kitty mixed-precision 2-bit KV cache library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method: "Kitty: Accurate and Efficient 2-bit KV Cache Quantization with
 * Dynamic Channel-wise Precision Boost" (arXiv 2511.18643), Abstract -- Key
 * channels are ranked by sensitivity and a small fraction is kept at higher
 * precision; each mixed-precision Key page is stored as two tensors of uniform
 * 2-bit codes inside a page-centric KV layout, so that dequantization is the
 * same for every lane.  The per-page arithmetic follows the VeloxQuant-MLX
 * documentation page "Kitty -- Dynamic Channel-wise Mixed-Precision Keys",
 * section "How it works / Prefill phase", steps 1-3 (channel variance over the
 * token axis, top hi_fraction x D channels at 4 bits, the rest at 2 bits,
 * asymmetric min/max over groups of 32 tokens), and its "Configuration
 * reference" (head_dim, hi_fraction, hi_bit = 4, lo_bit = 2, group_size = 32).
 *
 * Conventions for every entry point:
 *  - Return 0 (KITTY_OK) or a negative KITTY_ERR_* code.  On error,
 *    kitty_last_error() returns a message for the calling thread.  Argument
 *    validation happens before any HIP call, so an invalid argument never
 *    touches the device.
 *  - Every pointer named "device" is HIP device memory owned by the caller.
 *    The library allocates nothing, keeps no global mutable state besides the
 *    thread-local error text (and, for kitty_decode_step_noalloc, one static
 *    device array per GPU), and never synchronizes: all work is enqueued
 *    on `stream` (a hipStream_t; NULL = the default stream) and is
 *    asynchronous to the host.
 *  - fp16 arrays are IEEE binary16 passed as uint16_t.
 *  - Device-side contents (block-table entries, sequence lengths) are read by
 *    the kernels; a block-table entry outside [0, n_pages) makes the kernels
 *    skip that page (no access outside the pool), which leaves the result
 *    undefined but never faults.
 */
#ifndef KITTY_H
#define KITTY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KITTY_ABI_VERSION 3

enum {
  KITTY_OK = 0,
  KITTY_ERR_INVALID_ARG = -1, /* null pointer, negative/inconsistent size, misalignment */
  KITTY_ERR_UNSUPPORTED = -2, /* head_dim != 128, page_tokens != 32, bad n_hi, lo_bit or rank_mode */
  KITTY_ERR_WORKSPACE = -3,   /* workspace smaller than kitty_decode_workspace_bytes */
  KITTY_ERR_HIP = -4,         /* a kernel launch failed (hipGetLastError) */
  KITTY_ERR_NO_PAGES = -5     /* kitty_pool_reserve: the pool has too few free pages */
};

/* Cache geometry ("Configuration reference": head_dim, group_size,
 * hi_fraction, hi_bit, lo_bit; n_hi = hi_fraction * head_dim rounded half to
 * even).  Two bit-width pairs are supported, the two ends of the table
 * "Tuning avg_bits": (hi_bit, lo_bit) = (4, 2), the default, and (8, 4).  A
 * boosted Key code of hi_bit = 2 * lo_bit bits is stored as two lo_bit codes
 * (base = high half, boost = low half); Values use lo_bit. */
typedef struct {
  int32_t head_dim;    /* D; must be 128 */
  int32_t page_tokens; /* tokens per page = Key group size; must be 32 */
  int32_t n_kv_heads;  /* Hkv, 1..1024 */
  int32_t n_hi;        /* boosted channels per page, 0..D (any count) */
  int32_t lo_bit;      /* 2 (hi_bit 4) or 4 (hi_bit 8) */
  int32_t rank_mode;   /* KITTY_RANK_PAGE or KITTY_RANK_RUNNING */
} kitty_config_t;

/* Ranking modes (which channels of a page are boosted):
 *  KITTY_RANK_PAGE: by the page's own per-channel variance over its 32 tokens
 *    ("How it works / Prefill phase" steps 1-2 applied per page).
 *  KITTY_RANK_RUNNING: by the head's running variance ("How it works":
 *    Prefill step 1 over the whole prefill sequence, step 5 and "Decode
 *    phase" steps 1-2 running sums of k and k^2): prefill pages take the
 *    ranking over all prefill tokens of their sequence (tail included), a page
 *    sealed by an append the ranking over every token stored at that moment.
 *    The sums are exact (k * 2^24 is an integer for every fp16 k), so the
 *    ranking does not depend on the order of accumulation.  Needs
 *    kitty_kv_view_t.key_stats; at most 2^23 tokens per sequence. */
enum { KITTY_RANK_PAGE = 0, KITTY_RANK_RUNNING = 1 };

/* Bytes of running-mode state per (sequence, KV head): two copies of the
 * sums at bytes 0 and 3072, each int64 s1[128] (sum of k * 2^24), uint64
 * s2_lo[128] and s2_hi[128] (the 128-bit sum of (k * 2^24)^2); a sequence of
 * n tokens keeps its sums in copy n & 1.  Then uint32 mask[4] at byte 6144
 * (the ranking of the last prefill: channel c at bit c & 31 of word c >> 5)
 * and reserved bytes. */
#define KITTY_KEY_STATS_BYTES 8192

/* A paged cache (Abstract: page-centric KV layout).  One physical page holds
 * the records of all Hkv heads for 32 consecutive tokens of one sequence; the
 * block table maps (sequence b, logical page j) to a physical page id.
 * Record layout of one (page, head), with b = lo_bit and s = n_hi rounded up
 * to a multiple of 16 (boost slots; slots n_hi .. s-1 hold code 0 and index
 * 0): K base plane 512*b B, K boost plane 4*b*s B, V codes 512*b B, kscale
 * fp16[128], kmin fp16[128], vscale fp16[4][32], vmin fp16[4][32], idx
 * uint8[s] -- 1024*(b + 1) + (4*b + 1)*s bytes in total (3072 + 9*s at
 * lo_bit 2, 5120 + 17*s at lo_bit 4).  The code planes are 16*b-byte chunks, one per
 * lane of a 64-lane wave, of 32-bit words of 32/b codes each (the chunk and
 * bit placement is the one internal header kitty_internal.h documents).  Head
 * h's record starts at byte h * kitty_record_bytes; a physical page is
 * kitty_page_bytes long. */
typedef struct {
  void* pages;                /* device; n_pages * page_bytes bytes, 256-byte aligned */
  int64_t n_pages;            /* physical pages in the pool, >= 1 */
  const int32_t* block_table; /* device int32 [batch][max_pages] physical page ids */
  int32_t batch;              /* B >= 1 */
  int32_t max_pages;          /* block-table row length (logical pages per sequence), >= 1 */
  uint16_t* tail_k;           /* device fp16 [batch][Hkv][32][D]: the unsealed tail page */
  uint16_t* tail_v;           /* device fp16 [batch][Hkv][32][D] */
  int32_t* seq_lens;          /* device int32 [batch]: tokens stored (sealed pages + tail) */
  void* key_stats;            /* device [batch][Hkv][KITTY_KEY_STATS_BYTES], 16-byte aligned: running
                                 sums (KITTY_RANK_RUNNING only; ignored, may be NULL, otherwise).  Prefill
                                 writes them for the sequences it fills, append and the fused step add
                                 every appended token; their contents are only meaningful to this library */
} kitty_kv_view_t;

/* Version of this ABI (KITTY_ABI_VERSION). */
int kitty_abi_version(void);

/* Message for the last non-zero return on this thread ("" if none). */
const char* kitty_last_error(void);

/* Bytes of one (page, head) record: 1024 * (lo_bit + 1) + (4 * lo_bit + 1) * s,
 * s = n_hi rounded up to a multiple of 16. */
int kitty_record_bytes(const kitty_config_t* cfg, size_t* out);

/* Bytes of one physical page: n_kv_heads records, rounded up to 256. */
int kitty_page_bytes(const kitty_config_t* cfg, size_t* out);

/* Prefill ("How it works / Prefill phase", steps 1-3, per page of 32 tokens).
 * k, v: device fp16 [batch][Hkv][S][D], contiguous, 16-byte aligned.  For each
 * sequence b with
 * length n_b = (lens ? lens[b] : S), n_b <= S: the first floor(n_b / 32)
 * pages are ranked, quantized and packed into the physical pages
 * block_table[b][0..], the remaining n_b mod 32 tokens are copied verbatim
 * into tail_k / tail_v slots 0.., and seq_lens[b] = n_b.  lens: optional
 * device int32 [batch]; a negative lens[b] leaves sequence b untouched (no
 * page, tail or length written), so that one call can fill some slots of a
 * serving batch while the others keep decoding.  Requires floor(S / 32) <= max_pages.
 * KITTY_RANK_RUNNING: first the exact running sums over each filled
 * sequence's n_b tokens are written to its key_stats (replacing what was
 * there), then every page of the sequence is quantized with the ranking
 * they give; S <= 2^23. */
int kitty_quantize_pages(const kitty_config_t* cfg, const kitty_kv_view_t* kv,
                         const uint16_t* k, const uint16_t* v, int32_t S,
                         const int32_t* lens, void* stream);

/* Decode-time append of one token per sequence.  k_new, v_new: device fp16
 * [batch][Hkv][D], 16-byte aligned.  A sequence with seq_lens[b] < 0 is an
 * inactive slot and is skipped.  With n = seq_lens[b]: the token is stored in tail slot
 * n mod 32 and seq_lens[b] becomes n + 1; when that slot is the 32nd, the
 * full tail is quantized exactly like a prefill page and written to physical
 * page block_table[b][n / 32] (the tail page stays fp16 until it fills).  The
 * caller maps block_table[b][n / 32] to a free page before that append; a
 * seal with n / 32 >= max_pages is skipped.  KITTY_RANK_RUNNING: the token is
 * added to the sequence's key_stats first, and a sealed page takes the
 * ranking over all n + 1 tokens. */
int kitty_append_token(const kitty_config_t* cfg, const kitty_kv_view_t* kv,
                       const uint16_t* k_new, const uint16_t* v_new, void* stream);

/* Workspace bytes kitty_decode_attention and kitty_decode_step need for this
 * shape: split-KV partial results (m, l, O per query head and decode
 * workgroup), one arrival counter per (sequence, KV head, group of 4 query
 * heads), one per sequence, and a page record per (sequence, KV head, head
 * group beyond the first) for the fused step's seal.  max_seq_len: an upper bound on every seq_lens[b].  The
 * size never decreases as max_seq_len grows, so a workspace sized for the
 * largest bound serves every call with a smaller one. */
int kitty_decode_workspace_bytes(const kitty_config_t* cfg, int32_t batch, int32_t n_q_heads,
                                 int32_t max_seq_len, size_t* out);

/* The split plan decode attention and the fused step use for this shape on
 * a device with n_cus compute units (1..256; 0 = the current device): out[0]
 * = workgroups per (sequence, KV head, group of up to 4 query heads), out[1]
 * = waves per workgroup, out[2] = the largest workgroup the record size
 * allows.  Host only, for tests and tuning; the same validation and errors
 * as kitty_decode_workspace_bytes, and KITTY_ERR_HIP when n_cus = 0 finds no
 * device.  out: host int32[3]. */
int kitty_decode_plan(const kitty_config_t* cfg, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                      int32_t n_cus, int32_t* out);

/* Fused decode attention over the quantized cache (Abstract: page
 * dequantization fused into the decode kernels).  q: device fp16
 * [batch][Hq][D], 16-byte aligned, Hq a multiple of Hkv; query head hq reads KV head
 * hq / (Hq / Hkv).  For each sequence, attends over its first
 * n = min(seq_lens[b], max_seq_len) tokens -- sealed pages in order, then the
 * fp16 tail: out[b][hq] = softmax(q . k^ / sqrt(D)) . v^ with k^, v^ the
 * dequantized keys and values.  out: device fp32 [batch][Hq][D] (zeros for
 * an empty sequence or an inactive slot, seq_lens[b] < 0).  max_seq_len
 * sizes the split of the pages over the decode waves; tokens at or beyond it
 * are not attended (when it falls inside a sealed page, that page is
 * attended up to it); at most 131103 (4096 pages plus a tail), else
 * KITTY_ERR_UNSUPPORTED.
 * Inputs are finite fp16 (unchecked).  Every intermediate stays finite for
 * any finite q, K and V: the query is scaled by a power of two inside the
 * q * kscale limbs, and a page whose Value steps exceed 255.5 keeps its
 * softmax weights at most 1 (both exact in fp32).  Accuracy: the outputs
 * match fp32 attention over k^, v^ to about 2^-20 of max |v^| plus the
 * effect of that relative error on the logits (about 2^-21 |s|).
 * workspace: device, 256-byte
 * aligned, at least kitty_decode_workspace_bytes(...) bytes, zero-filled by
 * the caller before its first use (e.g. allocated zeroed); every completed
 * call leaves its counter area zero again, so one workspace serves any
 * number of calls, but calls that overlap in time must not share one. */
int kitty_decode_attention(const kitty_config_t* cfg, const kitty_kv_view_t* kv,
                           const uint16_t* q, int32_t n_q_heads, int32_t max_seq_len,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Fused decode step ("How it works / Decode phase" adapted to sealed pages;
 * Abstract: decode kernels fused with dequantization): exactly
 * kitty_append_token(k_new, v_new) followed by kitty_decode_attention(q), in
 * one launch.  The appended token is stored in tail slot n mod 32
 * (n = seq_lens[b] before the call); when it fills the tail page, that page
 * is quantized like a prefill page into block_table[b][n / 32] (skipped if
 * that entry is >= max_pages or outside the pool, as the append does) and
 * attended as a sealed page; seq_lens[b] becomes n + 1.  Inactive slots
 * (seq_lens[b] < 0) append nothing and attend nothing.  k_new, v_new:
 * device fp16 [batch][Hkv][D], 16-byte aligned.  The query attends the first
 * min(n + 1, max_seq_len) tokens.  Other arguments, the workspace (the same size
 * and zero-fill rules) and the errors are those of kitty_decode_attention.
 * The result equals the two separate calls' within floating-point rounding
 * (the page sealed by this call is folded in by another wave); the records,
 * tails, lengths and (KITTY_RANK_RUNNING) key_stats it writes are identical. */
int kitty_decode_step(const kitty_config_t* cfg, const kitty_kv_view_t* kv, const uint16_t* k_new,
                      const uint16_t* v_new, const uint16_t* q, int32_t n_q_heads, int32_t max_seq_len,
                      float* out, void* workspace, size_t workspace_bytes, void* stream);

/* The fused decode step for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid hipMalloc.  Exactly kitty_decode_step, except that the workspace is
 * the library's own: a static device array of KITTY_NOALLOC_SCRATCH_BYTES
 * per GPU, held from the first call on that GPU until the process ends.  It
 * allocates nothing (no hipMalloc, hipFree or allocating library call).  The
 * stream must belong to the current device.  Each call first clears the
 * arrival counters in that array with a small kernel on `stream` (so two
 * launches per call), then runs the decode step.  Every call on a GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams,
 * other threads) race and give undefined results; calls ordered on one
 * stream are safe.  A shape whose workspace (kitty_decode_workspace_bytes)
 * exceeds KITTY_NOALLOC_SCRATCH_BYTES returns KITTY_ERR_WORKSPACE before any
 * HIP call; the other errors are those of kitty_decode_step. */
#define KITTY_NOALLOC_SCRATCH_BYTES (16u << 20)
int kitty_decode_step_noalloc(const kitty_config_t* cfg, const kitty_kv_view_t* kv, const uint16_t* k_new,
                              const uint16_t* v_new, const uint16_t* q, int32_t n_q_heads, int32_t max_seq_len,
                              float* out, void* stream);

/* Page pool for ragged serving (the page-centric layout of the Abstract
 * lets sequences of any length share one pool).  Host only: these calls
 * touch no device memory and allocate nothing.  The caller owns the pool
 * struct, its free list and a host mirror of the block table, whose rows it
 * passes in; after a call that changes a row, the caller copies that row to
 * the device block table before the next kernel that reads it.  Unmapped
 * entries are -1.  Not thread-safe: one pool, one thread at a time. */
typedef struct {
  int32_t* free_list; /* host int32 [n_pages], caller-owned: entries [0, n_free) are free page ids */
  int64_t n_pages;    /* physical pages in the pool, 1 .. 2^31 - 1 */
  int64_t n_free;     /* free pages */
} kitty_pool_t;

/* Make every page of [0, n_pages) free; later reservations take pages 0, 1,
 * 2, ... in that order, and released pages are taken again first. */
int kitty_pool_init(kitty_pool_t* pool, int32_t* free_list, int64_t n_pages);

/* Map the pages a sequence needs to hold n_tokens tokens: entries
 * 0 .. floor(n_tokens / 32) - 1 of its row (the pages that its prefill, or
 * its appends up to that length, seal).  Call it with the length a prefill
 * or a decode step will reach, before that call.  All or nothing: with too
 * few free pages it returns KITTY_ERR_NO_PAGES and changes nothing.  row:
 * host int32 [max_pages]; every entry must be -1 or a page id below n_pages;
 * floor(n_tokens / 32) <= max_pages. */
int kitty_pool_reserve(kitty_pool_t* pool, int32_t* row, int32_t max_pages, int32_t n_tokens);

/* Return every mapped page of a row to the pool (e.g. when its sequence
 * ends); its entries become -1.  Releasing more pages than the pool holds
 * (a page released twice) is KITTY_ERR_INVALID_ARG, with nothing changed. */
int kitty_pool_release(kitty_pool_t* pool, int32_t* row, int32_t max_pages);

#ifdef __cplusplus
}
#endif

#endif /* KITTY_H */
