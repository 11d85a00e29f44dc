// C ABI of the Kitty library: argument validation (before any HIP call),
// layout sizes and kernel launches.  See include/kitty.h for the contract.
#include "../../include/kitty.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kitty_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return KITTY_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_config(const kitty_config_t* cfg) {
  if (!cfg) return fail(KITTY_ERR_INVALID_ARG, "cfg is null");
  if (cfg->head_dim != kitty::kHeadDim)
    return fail(KITTY_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", cfg->head_dim);
  if (cfg->page_tokens != kitty::kPageTokens)
    return fail(KITTY_ERR_UNSUPPORTED, "page_tokens %d unsupported (only 32)", cfg->page_tokens);
  if (cfg->n_kv_heads < 1 || cfg->n_kv_heads > 1024)
    return fail(KITTY_ERR_INVALID_ARG, "n_kv_heads %d out of range [1, 1024]", cfg->n_kv_heads);
  if (cfg->n_hi < 0 || cfg->n_hi > cfg->head_dim)
    return fail(KITTY_ERR_UNSUPPORTED, "n_hi %d unsupported (0 to 128)", cfg->n_hi);
  if (cfg->lo_bit != 2 && cfg->lo_bit != 4)
    return fail(KITTY_ERR_UNSUPPORTED, "lo_bit %d unsupported (2 or 4)", cfg->lo_bit);
  if (cfg->rank_mode != KITTY_RANK_PAGE && cfg->rank_mode != KITTY_RANK_RUNNING)
    return fail(KITTY_ERR_UNSUPPORTED, "rank_mode %d unsupported (KITTY_RANK_PAGE or KITTY_RANK_RUNNING)",
                cfg->rank_mode);
  return KITTY_OK;
}

int check_view(const kitty_config_t* cfg, const kitty_kv_view_t* kv) {
  if (!kv) return fail(KITTY_ERR_INVALID_ARG, "kv view is null");
  if (!kv->pages || !aligned(kv->pages, 256)) return fail(KITTY_ERR_INVALID_ARG, "pages null or not 256-byte aligned");
  if (kv->n_pages < 1) return fail(KITTY_ERR_INVALID_ARG, "n_pages must be >= 1");
  if (!kv->block_table || !aligned(kv->block_table, 4)) return fail(KITTY_ERR_INVALID_ARG, "block_table null or misaligned");
  if (kv->batch < 1 || kv->batch > 65535) return fail(KITTY_ERR_INVALID_ARG, "batch %d out of range [1, 65535]", kv->batch);
  if (kv->max_pages < 1) return fail(KITTY_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (!kv->tail_k || !kv->tail_v || !aligned(kv->tail_k, 16) || !aligned(kv->tail_v, 16))
    return fail(KITTY_ERR_INVALID_ARG, "tail_k / tail_v null or not 16-byte aligned");
  if (!kv->seq_lens || !aligned(kv->seq_lens, 4)) return fail(KITTY_ERR_INVALID_ARG, "seq_lens null or misaligned");
  if (cfg->rank_mode == KITTY_RANK_RUNNING && (!kv->key_stats || !aligned(kv->key_stats, 16)))
    return fail(KITTY_ERR_INVALID_ARG, "the running ranking mode needs key_stats, 16-byte aligned");
  return KITTY_OK;
}

// the running sums of a (sequence, KV head), or null in the page ranking mode
uint8_t* key_stats_of(const kitty_config_t* cfg, const kitty_kv_view_t* kv) {
  return cfg->rank_mode == KITTY_RANK_RUNNING ? static_cast<uint8_t*>(kv->key_stats) : nullptr;
}

int check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KITTY_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int kitty_abi_version(void) { return KITTY_ABI_VERSION; }

const char* kitty_last_error(void) { return g_last_error.c_str(); }

int kitty_record_bytes(const kitty_config_t* cfg, size_t* out) {
  if (int r = check_config(cfg)) return r;
  if (!out) return fail(KITTY_ERR_INVALID_ARG, "out is null");
  *out = (size_t)kitty::rec_bytes(kitty::boost_slots(cfg->n_hi), cfg->lo_bit);
  return ok();
}

int kitty_page_bytes(const kitty_config_t* cfg, size_t* out) {
  if (int r = check_config(cfg)) return r;
  if (!out) return fail(KITTY_ERR_INVALID_ARG, "out is null");
  *out = (size_t)kitty::page_stride_bytes(cfg->n_kv_heads, cfg->n_hi, cfg->lo_bit);
  return ok();
}

int kitty_quantize_pages(const kitty_config_t* cfg, const kitty_kv_view_t* kv, const uint16_t* k,
                         const uint16_t* v, int32_t S, const int32_t* lens, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_view(cfg, kv)) return r;
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16)) return fail(KITTY_ERR_INVALID_ARG, "k / v null or not 16-byte aligned");
  if (S < 0) return fail(KITTY_ERR_INVALID_ARG, "S must be >= 0");
  if (S / kitty::kPageTokens > kv->max_pages)
    return fail(KITTY_ERR_INVALID_ARG, "S / 32 = %d exceeds max_pages %d", S / kitty::kPageTokens, kv->max_pages);
  if (lens && !aligned(lens, 4)) return fail(KITTY_ERR_INVALID_ARG, "lens misaligned");
  if (cfg->rank_mode == KITTY_RANK_RUNNING && S > kitty::kMaxRunningTokens)
    return fail(KITTY_ERR_UNSUPPORTED, "S %d exceeds %d tokens in the running ranking mode", S, kitty::kMaxRunningTokens);
  kitty::QuantizeParams p{};
  p.pages = static_cast<uint8_t*>(kv->pages);
  p.n_pages = kv->n_pages;
  p.page_bytes = kitty::page_stride_bytes(cfg->n_kv_heads, cfg->n_hi, cfg->lo_bit);
  p.block_table = kv->block_table;
  p.max_pages = kv->max_pages;
  p.batch = kv->batch;
  p.n_kv_heads = cfg->n_kv_heads;
  p.n_hi = cfg->n_hi;
  p.lo_bit = cfg->lo_bit;
  p.tail_k = reinterpret_cast<_Float16*>(kv->tail_k);
  p.tail_v = reinterpret_cast<_Float16*>(kv->tail_v);
  p.seq_lens = kv->seq_lens;
  p.k = reinterpret_cast<const _Float16*>(k);
  p.v = reinterpret_cast<const _Float16*>(v);
  p.S = S;
  p.lens = lens;
  p.key_stats = key_stats_of(cfg, kv);
  (void)hipGetLastError();
  return check_launch(kitty::launch_quantize(p, static_cast<hipStream_t>(stream)), "quantize_pages");
}

int kitty_append_token(const kitty_config_t* cfg, const kitty_kv_view_t* kv, const uint16_t* k_new,
                       const uint16_t* v_new, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_view(cfg, kv)) return r;
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(KITTY_ERR_INVALID_ARG, "k_new / v_new null or not 16-byte aligned");
  kitty::AppendParams p{};
  p.pages = static_cast<uint8_t*>(kv->pages);
  p.n_pages = kv->n_pages;
  p.page_bytes = kitty::page_stride_bytes(cfg->n_kv_heads, cfg->n_hi, cfg->lo_bit);
  p.block_table = kv->block_table;
  p.max_pages = kv->max_pages;
  p.batch = kv->batch;
  p.n_kv_heads = cfg->n_kv_heads;
  p.n_hi = cfg->n_hi;
  p.lo_bit = cfg->lo_bit;
  p.tail_k = reinterpret_cast<_Float16*>(kv->tail_k);
  p.tail_v = reinterpret_cast<_Float16*>(kv->tail_v);
  p.seq_lens = kv->seq_lens;
  p.k_new = reinterpret_cast<const _Float16*>(k_new);
  p.v_new = reinterpret_cast<const _Float16*>(v_new);
  p.key_stats = key_stats_of(cfg, kv);
  (void)hipGetLastError();
  return check_launch(kitty::launch_append(p, static_cast<hipStream_t>(stream)), "append_token");
}

// Workspace of decode attention and the fused decode step, in order:
// per-workgroup partials, workgroup arrival counters, per-sequence arrival
// counters, and the records that head groups >= 1 re-quantize at a seal.
struct DecodeWorkspace {
  size_t partials, counters, seq_counters, seal_scratch, total;
};

// The plan for `cus` compute units; the workspace layout always for
// kitty::kMaxCus, whose plan needs at least as many workgroups (the plan is
// non-decreasing in the CU count), so one workspace size serves every device.
static int decode_shape(const kitty_config_t* cfg, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                        int cus, kitty::SplitPlan* plan, int* n_head_groups, DecodeWorkspace* ws) {
  if (batch < 1 || batch > 65535) return fail(KITTY_ERR_INVALID_ARG, "batch %d out of range [1, 65535]", batch);
  if (n_q_heads < 1 || n_q_heads % cfg->n_kv_heads != 0)
    return fail(KITTY_ERR_INVALID_ARG, "n_q_heads %d must be a positive multiple of n_kv_heads %d", n_q_heads,
                cfg->n_kv_heads);
  if (max_seq_len < 0) return fail(KITTY_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (max_seq_len > kitty::kMaxSeqLen)
    return fail(KITTY_ERR_UNSUPPORTED, "max_seq_len %d exceeds %d", max_seq_len, kitty::kMaxSeqLen);
  const int G = n_q_heads / cfg->n_kv_heads;
  *n_head_groups = (G + 3) / 4;
  if ((long)cfg->n_kv_heads * *n_head_groups > 65535) return fail(KITTY_ERR_INVALID_ARG, "too many heads");
  const int wmax = kitty::decode_max_wg_waves(cfg->n_hi, cfg->lo_bit);
  *plan = kitty::plan_splits(batch, cfg->n_kv_heads, *n_head_groups, max_seq_len, wmax, cus);
  const kitty::SplitPlan widest = kitty::plan_splits(batch, cfg->n_kv_heads, *n_head_groups, max_seq_len, wmax,
                                                     kitty::kMaxCus);
  auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t part = (size_t)batch * n_q_heads * widest.n_wg * kitty::kPartialStride * sizeof(float);
  const size_t cnt = (size_t)batch * cfg->n_kv_heads * *n_head_groups * sizeof(int);
  const size_t seqc = (size_t)batch * kitty::kSeqCounterStride * sizeof(int);
  const size_t seal = (size_t)batch * cfg->n_kv_heads * (*n_head_groups - 1) * kitty::rec_bytes(kitty::boost_slots(cfg->n_hi), cfg->lo_bit);
  ws->partials = 0;
  ws->counters = r256(part);
  ws->seq_counters = ws->counters + r256(cnt);
  ws->seal_scratch = ws->seq_counters + r256(seqc);
  ws->total = ws->seal_scratch + r256(seal);
  return KITTY_OK;
}

int kitty_decode_workspace_bytes(const kitty_config_t* cfg, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                                 size_t* out) {
  if (int r = check_config(cfg)) return r;
  if (!out) return fail(KITTY_ERR_INVALID_ARG, "out is null");
  kitty::SplitPlan plan;
  int nhg;
  DecodeWorkspace ws;
  if (int r = decode_shape(cfg, batch, n_q_heads, max_seq_len, kitty::kMaxCus, &plan, &nhg, &ws)) return r;
  *out = ws.total;
  return ok();
}

// Compute units of the device a stream runs on (at most kitty::kMaxCus), or
// 0 on failure.
static int stream_cus(hipStream_t stream) {
  int dev = 0, cus = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess && hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 0;
  return cus < kitty::kMaxCus ? cus : kitty::kMaxCus;
}

int kitty_decode_plan(const kitty_config_t* cfg, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                      int32_t n_cus, int32_t* out) {
  if (int r = check_config(cfg)) return r;
  if (!out) return fail(KITTY_ERR_INVALID_ARG, "out is null");
  if (n_cus < 0 || n_cus > kitty::kMaxCus) return fail(KITTY_ERR_INVALID_ARG, "n_cus %d out of range [0, %d]", n_cus, kitty::kMaxCus);
  kitty::SplitPlan plan;
  int nhg;
  DecodeWorkspace ws;
  if (int r = decode_shape(cfg, batch, n_q_heads, max_seq_len, kitty::kMaxCus, &plan, &nhg, &ws)) return r;
  int cus = n_cus;
  if (cus == 0 && (cus = stream_cus(nullptr)) == 0) return fail(KITTY_ERR_HIP, "no device to read the compute unit count from");
  if (int r = decode_shape(cfg, batch, n_q_heads, max_seq_len, cus, &plan, &nhg, &ws)) return r;
  out[0] = plan.n_wg;
  out[1] = plan.wg_waves;
  out[2] = kitty::decode_max_wg_waves(cfg->n_hi, cfg->lo_bit);
  return ok();
}

// Shared by kitty_decode_attention (k_new == v_new == null) and
// kitty_decode_step.
static int decode_launch(const kitty_config_t* cfg, const kitty_kv_view_t* kv, const uint16_t* k_new,
                         const uint16_t* v_new, const uint16_t* q, int32_t n_q_heads, int32_t max_seq_len,
                         float* out, void* workspace, size_t workspace_bytes, void* stream, const char* what) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_view(cfg, kv)) return r;
  if (!q || !aligned(q, 16)) return fail(KITTY_ERR_INVALID_ARG, "q null or not 16-byte aligned");
  if (!out || !aligned(out, 4)) return fail(KITTY_ERR_INVALID_ARG, "out null or misaligned");
  kitty::SplitPlan plan;
  int nhg;
  DecodeWorkspace ws;
  if (int r = decode_shape(cfg, kv->batch, n_q_heads, max_seq_len, kitty::kMaxCus, &plan, &nhg, &ws)) return r;
  if (!workspace || !aligned(workspace, 256)) return fail(KITTY_ERR_INVALID_ARG, "workspace null or not 256-byte aligned");
  if (workspace_bytes < ws.total)
    return fail(KITTY_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, ws.total);
  const int cus = stream_cus(static_cast<hipStream_t>(stream));
  if (cus == 0) return fail(KITTY_ERR_HIP, "cannot read the compute unit count of the stream's device");
  if (cus != kitty::kMaxCus && decode_shape(cfg, kv->batch, n_q_heads, max_seq_len, cus, &plan, &nhg, &ws)) return KITTY_ERR_INVALID_ARG;
  uint8_t* wsb = static_cast<uint8_t*>(workspace);
  kitty::DecodeParams p{};
  p.pages = static_cast<uint8_t*>(kv->pages);
  p.n_pages = kv->n_pages;
  p.page_bytes = kitty::page_stride_bytes(cfg->n_kv_heads, cfg->n_hi, cfg->lo_bit);
  p.block_table = kv->block_table;
  p.max_pages = kv->max_pages;
  p.batch = kv->batch;
  p.n_kv_heads = cfg->n_kv_heads;
  p.n_hi = cfg->n_hi;
  p.lo_bit = cfg->lo_bit;
  p.tail_k = reinterpret_cast<_Float16*>(kv->tail_k);
  p.tail_v = reinterpret_cast<_Float16*>(kv->tail_v);
  p.seq_lens = kv->seq_lens;
  p.q = reinterpret_cast<const _Float16*>(q);
  p.k_new = reinterpret_cast<const _Float16*>(k_new);
  p.v_new = reinterpret_cast<const _Float16*>(v_new);
  p.n_q_heads = n_q_heads;
  p.group = n_q_heads / cfg->n_kv_heads;
  p.n_head_groups = nhg;
  p.max_seq_len = max_seq_len;
  p.n_wg = plan.n_wg;
  p.wg_waves = plan.wg_waves;
  p.partial = reinterpret_cast<float*>(wsb + ws.partials);
  p.counters = reinterpret_cast<int*>(wsb + ws.counters);
  p.seq_counters = reinterpret_cast<int*>(wsb + ws.seq_counters);
  p.seal_scratch = wsb + ws.seal_scratch;
  p.out = out;
  p.key_stats = key_stats_of(cfg, kv);
  (void)hipGetLastError();
  return check_launch(kitty::launch_decode(p, static_cast<hipStream_t>(stream)), what);
}

int kitty_decode_attention(const kitty_config_t* cfg, const kitty_kv_view_t* kv, const uint16_t* q,
                           int32_t n_q_heads, int32_t max_seq_len, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return decode_launch(cfg, kv, nullptr, nullptr, q, n_q_heads, max_seq_len, out, workspace, workspace_bytes,
                       stream, "decode_attention");
}

int kitty_decode_step(const kitty_config_t* cfg, const kitty_kv_view_t* kv, const uint16_t* k_new,
                      const uint16_t* v_new, const uint16_t* q, int32_t n_q_heads, int32_t max_seq_len,
                      float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(KITTY_ERR_INVALID_ARG, "k_new / v_new null or not 16-byte aligned");
  return decode_launch(cfg, kv, k_new, v_new, q, n_q_heads, max_seq_len, out, workspace, workspace_bytes, stream,
                       "decode_step");
}

}  // extern "C"

// ---- the fused step without a caller workspace -----------------------------------
// The decode workspace of kitty_decode_step_noalloc (split partials, arrival
// counters, seal records) lives in this array, one copy per GPU, held until
// the process ends.  Host code never uses its name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[KITTY_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // the device address of `scratch` on each device, once looked up

// The device address of `scratch` on device `dev` (the current device).
int scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KITTY_ERR_HIP, "hipGetSymbolAddress of the decode scratch failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KITTY_OK;
}
}  // namespace

extern "C" {

int kitty_decode_step_noalloc(const kitty_config_t* cfg, const kitty_kv_view_t* kv, const uint16_t* k_new,
                              const uint16_t* v_new, const uint16_t* q, int32_t n_q_heads, int32_t max_seq_len,
                              float* out, void* stream) {
  // every argument and the scratch size are checked before any HIP call
  if (int r = check_config(cfg)) return r;
  if (int r = check_view(cfg, kv)) return r;
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(KITTY_ERR_INVALID_ARG, "k_new / v_new null or not 16-byte aligned");
  if (!q || !aligned(q, 16)) return fail(KITTY_ERR_INVALID_ARG, "q null or not 16-byte aligned");
  if (!out || !aligned(out, 4)) return fail(KITTY_ERR_INVALID_ARG, "out null or misaligned");
  kitty::SplitPlan plan;
  int nhg;
  DecodeWorkspace ws;
  if (int r = decode_shape(cfg, kv->batch, n_q_heads, max_seq_len, kitty::kMaxCus, &plan, &nhg, &ws)) return r;
  if (ws.total > KITTY_NOALLOC_SCRATCH_BYTES)
    return fail(KITTY_ERR_WORKSPACE, "this shape needs %zu bytes of decode scratch, more than the %zu the "
                "allocation-free step holds (use kitty_decode_step with a workspace)", ws.total,
                (size_t)KITTY_NOALLOC_SCRATCH_BYTES);
  int dev = -1, sdev = -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(KITTY_ERR_HIP, "no current device (or device id beyond %d)", kMaxDevices - 1);
  if (hipStreamGetDevice(s, &sdev) == hipSuccess && sdev != dev)
    return fail(KITTY_ERR_INVALID_ARG, "the stream belongs to device %d, not the current device %d", sdev, dev);
  void* ptr = nullptr;
  if (int r = scratch_on(dev, &ptr)) return r;
  // the arrival counters start at zero: clear them (a completed call also
  // leaves them zero, but the layout moves with the shape)
  uint8_t* base = static_cast<uint8_t*>(ptr);
  (void)hipGetLastError();
  const hipError_t e = kitty::launch_zero_words(reinterpret_cast<uint32_t*>(base + ws.counters),
                                                (ws.seal_scratch - ws.counters) / 4, s);
  if (e != hipSuccess) return fail(KITTY_ERR_HIP, "decode scratch clear failed: %s", hipGetErrorString(e));
  return decode_launch(cfg, kv, k_new, v_new, q, n_q_heads, max_seq_len, out, ptr, KITTY_NOALLOC_SCRATCH_BYTES,
                       stream, "decode_step_noalloc");
}


// ---- page pool (host only) -------------------------------------------------------

int kitty_pool_init(kitty_pool_t* pool, int32_t* free_list, int64_t n_pages) {
  if (!pool || !free_list) return fail(KITTY_ERR_INVALID_ARG, "pool or free_list is null");
  if (n_pages < 1 || n_pages > 0x7FFFFFFF) return fail(KITTY_ERR_INVALID_ARG, "n_pages %lld out of range", (long long)n_pages);
  for (int64_t i = 0; i < n_pages; ++i) free_list[i] = (int32_t)(n_pages - 1 - i);  // the stack top is page 0
  pool->free_list = free_list;
  pool->n_pages = n_pages;
  pool->n_free = n_pages;
  return ok();
}

}  // extern "C"

static int check_pool(const kitty_pool_t* pool, const int32_t* row, int32_t max_pages) {
  if (!pool || !pool->free_list || !row) return fail(KITTY_ERR_INVALID_ARG, "pool, its free list or row is null");
  if (pool->n_pages < 1 || pool->n_pages > 0x7FFFFFFF || pool->n_free < 0 || pool->n_free > pool->n_pages)
    return fail(KITTY_ERR_INVALID_ARG, "pool state is inconsistent");
  if (max_pages < 1) return fail(KITTY_ERR_INVALID_ARG, "max_pages must be >= 1");
  for (int32_t j = 0; j < max_pages; ++j)
    if (row[j] < -1 || row[j] >= pool->n_pages)
      return fail(KITTY_ERR_INVALID_ARG, "row entry %d = %d is neither -1 nor a page id", j, row[j]);
  return KITTY_OK;
}

extern "C" {

int kitty_pool_reserve(kitty_pool_t* pool, int32_t* row, int32_t max_pages, int32_t n_tokens) {
  if (int r = check_pool(pool, row, max_pages)) return r;
  if (n_tokens < 0) return fail(KITTY_ERR_INVALID_ARG, "n_tokens must be >= 0");
  const int32_t need = n_tokens / kitty::kPageTokens;
  if (need > max_pages) return fail(KITTY_ERR_INVALID_ARG, "%d tokens need %d pages > max_pages %d", n_tokens, need, max_pages);
  int64_t missing = 0;
  for (int32_t j = 0; j < need; ++j) missing += row[j] < 0;
  if (missing > pool->n_free)
    return fail(KITTY_ERR_NO_PAGES, "%lld pages needed, %lld free", (long long)missing, (long long)pool->n_free);
  for (int32_t j = 0; j < need; ++j)
    if (row[j] < 0) row[j] = pool->free_list[--pool->n_free];
  return ok();
}

int kitty_pool_release(kitty_pool_t* pool, int32_t* row, int32_t max_pages) {
  if (int r = check_pool(pool, row, max_pages)) return r;
  int64_t mapped = 0;
  for (int32_t j = 0; j < max_pages; ++j) mapped += row[j] >= 0;
  if (pool->n_free + mapped > pool->n_pages)
    return fail(KITTY_ERR_INVALID_ARG, "releasing %lld pages overflows the pool (a page released twice?)", (long long)mapped);
  for (int32_t j = 0; j < max_pages; ++j)
    if (row[j] >= 0) {
      pool->free_list[pool->n_free++] = row[j];
      row[j] = -1;
    }
  return ok();
}

}  // extern "C"
