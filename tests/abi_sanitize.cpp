// Host-side exercise of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_abi_sanitize.py with the
// sanitizers on the host code only; no GPU, no kernel launch).  It walks the
// argument validation of every entry point, the size and split-plan
// arithmetic over a grid of shapes, and the page pool against a plain model,
// so that an out-of-bounds access, an overflow or a misaligned access in any
// of those host paths stops the run.  Prints "ok <checks>" on success.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kitty.h"
#include "kitty_bench.h"

static long g_checks = 0;

#define CHECK(cond)                                                            \
  do {                                                                         \
    ++g_checks;                                                                \
    if (!(cond)) {                                                             \
      std::fprintf(stderr, "check failed at line %d: %s (last error: %s)\n",  \
                   __LINE__, #cond, kitty_last_error());                       \
      std::exit(1);                                                            \
    }                                                                          \
  } while (0)

static kitty_config_t config(int hkv, int n_hi, int lo_bit = 2, int rank = KITTY_RANK_PAGE) {
  kitty_config_t c{128, 32, hkv, n_hi, lo_bit, rank};
  return c;
}

// Tiny deterministic generator for the pool walk (splitmix64).
static uint64_t g_state = 0x243F6A8885A308D3ull;
static uint64_t next_u64() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static void config_validation() {
  size_t out = 0;
  CHECK(kitty_record_bytes(nullptr, &out) == KITTY_ERR_INVALID_ARG);
  kitty_config_t c = config(8, 32);
  CHECK(kitty_record_bytes(&c, nullptr) == KITTY_ERR_INVALID_ARG);
  const int bad[][6] = {{64, 32, 8, 32, 2, 0},  {128, 16, 8, 32, 2, 0}, {128, 32, 0, 32, 2, 0},
                        {128, 32, 1025, 32, 2, 0}, {128, 32, 8, -1, 2, 0}, {128, 32, 8, 129, 2, 0},
                        {128, 32, 8, 32, 3, 0},  {128, 32, 8, 32, 2, 2},  {128, 32, 8, 32, 2, -1}};
  for (const auto& b : bad) {
    kitty_config_t x{b[0], b[1], b[2], b[3], b[4], b[5]};
    CHECK(kitty_record_bytes(&x, &out) < 0);
    CHECK(kitty_page_bytes(&x, &out) < 0);
    CHECK(kitty_last_error()[0] != '\0');
  }
  for (int lo : {2, 4})
    for (int n_hi = 0; n_hi <= 128; ++n_hi)
      for (int hkv : {1, 7, 8, 1024}) {
        kitty_config_t x = config(hkv, n_hi, lo);
        size_t rb = 0, pb = 0;
        CHECK(kitty_record_bytes(&x, &rb) == KITTY_OK);
        CHECK(kitty_page_bytes(&x, &pb) == KITTY_OK);
        const size_t s = (size_t)(n_hi + 15) / 16 * 16;
        CHECK(rb == 1024u * (lo + 1) + (4u * lo + 1) * s);
        CHECK(pb % 256 == 0 && pb >= rb * hkv && pb < rb * hkv + 256);
      }
}

static void workspace_and_plan() {
  size_t ws = 0;
  int32_t plan[3] = {0, 0, 0};
  kitty_config_t c = config(8, 32);
  CHECK(kitty_decode_workspace_bytes(&c, 0, 32, 4096, &ws) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_decode_workspace_bytes(&c, 4, 30, 4096, &ws) == KITTY_ERR_INVALID_ARG);  // not a multiple of Hkv
  CHECK(kitty_decode_workspace_bytes(&c, 4, 32, -1, &ws) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_decode_workspace_bytes(&c, 4, 32, 131104, &ws) == KITTY_ERR_UNSUPPORTED);
  CHECK(kitty_decode_workspace_bytes(&c, 4, 32, 4096, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_decode_plan(&c, 4, 32, 4096, 257, plan) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_decode_plan(&c, 4, 32, 4096, -1, plan) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_decode_plan(&c, 4, 32, 4096, 256, nullptr) == KITTY_ERR_INVALID_ARG);
  // every plan the planner can make on a grid of shapes: sizes positive,
  // workspace monotone in the length bound
  for (int lo : {2, 4})
    for (int n_hi : {0, 13, 32, 100, 128})
      for (int hkv : {1, 8, 32})
        for (int group : {1, 2, 4, 5, 8})
          for (int batch : {1, 3, 16, 128, 1024})
            for (int cus : {1, 80, 256}) {
              kitty_config_t x = config(hkv, n_hi, lo);
              size_t prev = 0;
              for (int msl : {0, 1, 31, 32, 33, 4096, 32768, 131103}) {
                size_t w = 0;
                CHECK(kitty_decode_workspace_bytes(&x, batch, group * hkv, msl, &w) == KITTY_OK);
                CHECK(w >= prev && w % 256 == 0);
                prev = w;
                CHECK(kitty_decode_plan(&x, batch, group * hkv, msl, cus, plan) == KITTY_OK);
                CHECK(plan[0] >= 1 && plan[1] >= 2 && plan[1] <= plan[2] && plan[2] <= 12);
              }
            }
}

static void entry_validation() {
  kitty_config_t c = config(8, 32);
  alignas(256) static uint8_t pages[4096];
  static int32_t table[16];
  alignas(16) static uint16_t tail_k[64], tail_v[64], q[64];
  static int32_t lens[4];
  alignas(256) static uint8_t ws[1024];
  static float out[64];
  kitty_kv_view_t kv{pages, 1, table, 1, 1, tail_k, tail_v, lens, nullptr};
  // null and misaligned arguments fail before any device call
  CHECK(kitty_quantize_pages(&c, nullptr, tail_k, tail_v, 32, nullptr, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_quantize_pages(&c, &kv, nullptr, tail_v, 32, nullptr, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_quantize_pages(&c, &kv, tail_k, tail_v, -1, nullptr, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_append_token(&c, &kv, nullptr, tail_v, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_append_token(&c, &kv, reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(tail_k) + 2), tail_v,
                           nullptr) == KITTY_ERR_INVALID_ARG);
  kitty_kv_view_t bad = kv;
  bad.pages = pages + 16;
  CHECK(kitty_append_token(&c, &bad, tail_k, tail_v, nullptr) == KITTY_ERR_INVALID_ARG);
  bad = kv;
  bad.n_pages = 0;
  CHECK(kitty_append_token(&c, &bad, tail_k, tail_v, nullptr) == KITTY_ERR_INVALID_ARG);
  bad = kv;
  bad.batch = 0;
  CHECK(kitty_append_token(&c, &bad, tail_k, tail_v, nullptr) == KITTY_ERR_INVALID_ARG);
  bad = kv;
  bad.seq_lens = nullptr;
  CHECK(kitty_append_token(&c, &bad, tail_k, tail_v, nullptr) == KITTY_ERR_INVALID_ARG);
  kitty_config_t run = config(8, 32, 2, KITTY_RANK_RUNNING);
  CHECK(kitty_append_token(&run, &kv, tail_k, tail_v, nullptr) == KITTY_ERR_INVALID_ARG);  // key_stats missing
  CHECK(kitty_decode_attention(&c, &kv, q, 32, 64, nullptr, ws, sizeof ws, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_decode_attention(&c, &kv, q, 33, 64, out, ws, sizeof ws, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_decode_attention(&c, &kv, q, 32, 64, out, ws, 16, nullptr) == KITTY_ERR_WORKSPACE);
  CHECK(kitty_decode_attention(&c, &kv, q, 32, 64, out, ws + 16, sizeof ws - 16, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_decode_step(&c, &kv, nullptr, tail_v, q, 32, 64, out, ws, sizeof ws, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_decode_step(&c, &kv, tail_k, tail_v, q, 32, 200000, out, ws, sizeof ws, nullptr) ==
        KITTY_ERR_UNSUPPORTED);
  // a shape whose workspace exceeds the static scratch: rejected before any HIP call
  kitty_kv_view_t big = kv;
  big.batch = 65535;
  CHECK(kitty_decode_step_noalloc(&c, &big, tail_k, tail_v, q, 32, 131103, out, nullptr) == KITTY_ERR_WORKSPACE);
  CHECK(kitty_decode_step_noalloc(&c, &kv, nullptr, tail_v, q, 32, 64, out, nullptr) == KITTY_ERR_INVALID_ARG);
  uint32_t sink[4];
  CHECK(kitty_read_ceiling(nullptr, 1 << 20, KITTY_READ_VGPR, 8, 2, sink, 4, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_read_ceiling(pages, 4001, KITTY_READ_VGPR, 8, 2, sink, 4, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_read_ceiling(pages, 4096, KITTY_READ_VGPR, 6, 2, sink, 4, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_read_ceiling(pages, 4096, KITTY_READ_LDS_RECORDS, 13, 4, sink, 4, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_read_ceiling(pages, 4096, 7, 8, 2, sink, 4, nullptr) == KITTY_ERR_INVALID_ARG);
  alignas(256) static uint8_t other[4096];  // a destination apart from the source
  CHECK(kitty_stream_ceiling(nullptr, other, 4, 2048, 2048, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_stream_ceiling(pages, other, 4, 3000, 2048, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_stream_ceiling(pages, other, 4, 2048, 2000, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_stream_ceiling(pages, other, 0, 2048, 2048, nullptr) == KITTY_ERR_INVALID_ARG);
  CHECK(kitty_stream_ceiling(pages, pages + 2048, 4, 2048, 2048, nullptr) == KITTY_ERR_INVALID_ARG);  // overlap
  CHECK(kitty_stream_ceiling(pages, other, (int64_t)1 << 40, 65536, 65536, nullptr) == KITTY_ERR_INVALID_ARG);
}

// The pool against a plain model: the set of free pages and each row's
// mapped pages, over a random walk of reservations and releases.
static void pool_walk() {
  kitty_pool_t pool{};
  CHECK(kitty_pool_init(nullptr, nullptr, 4) == KITTY_ERR_INVALID_ARG);
  std::vector<int32_t> bad_list(2);
  CHECK(kitty_pool_init(&pool, bad_list.data(), 0) == KITTY_ERR_INVALID_ARG);
  const int n_pages = 97, rows = 6, max_pages = 40;
  std::vector<int32_t> free_list(n_pages);
  CHECK(kitty_pool_init(&pool, free_list.data(), n_pages) == KITTY_OK);
  CHECK(pool.n_free == n_pages);
  std::vector<std::vector<int32_t>> table(rows, std::vector<int32_t>(max_pages, -1));
  std::vector<int> owner(n_pages, -1);  // model: row owning each page
  for (int step = 0; step < 20000; ++step) {
    const int r = (int)(next_u64() % rows);
    if (next_u64() % 4 == 0) {
      CHECK(kitty_pool_release(&pool, table[r].data(), max_pages) == KITTY_OK);
      for (int p = 0; p < n_pages; ++p)
        if (owner[p] == r) owner[p] = -1;
      for (int j = 0; j < max_pages; ++j) CHECK(table[r][j] == -1);
    } else {
      const int32_t n_tok = (int32_t)(next_u64() % (32 * max_pages + 40));
      const int32_t need = n_tok / 32;
      long missing = 0;
      if (need <= max_pages)
        for (int j = 0; j < need; ++j) missing += table[r][j] < 0;
      const long free_before = pool.n_free;
      const std::vector<int32_t> before = table[r];
      const int rc = kitty_pool_reserve(&pool, table[r].data(), max_pages, n_tok);
      if (need > max_pages) {
        CHECK(rc == KITTY_ERR_INVALID_ARG && table[r] == before);
      } else if (missing > free_before) {
        CHECK(rc == KITTY_ERR_NO_PAGES && table[r] == before && pool.n_free == free_before);
      } else {
        CHECK(rc == KITTY_OK && pool.n_free == free_before - missing);
        for (int j = 0; j < need; ++j) {
          const int32_t p = table[r][j];
          CHECK(p >= 0 && p < n_pages);
          if (before[j] < 0) {
            CHECK(owner[p] == -1);
            owner[p] = r;
          } else {
            CHECK(p == before[j] && owner[p] == r);
          }
        }
      }
    }
    long owned = 0;
    for (int p = 0; p < n_pages; ++p) owned += owner[p] >= 0;
    CHECK(owned + pool.n_free == n_pages);
  }
  // a row entry outside the pool, and a double release, are rejected unchanged
  std::vector<int32_t> row(max_pages, -1);
  row[3] = n_pages;
  CHECK(kitty_pool_reserve(&pool, row.data(), max_pages, 64) == KITTY_ERR_INVALID_ARG);
  for (int r = 0; r < rows; ++r) CHECK(kitty_pool_release(&pool, table[r].data(), max_pages) == KITTY_OK);
  CHECK(pool.n_free == n_pages);
  std::vector<int32_t> stale(max_pages, -1);
  stale[0] = 5;
  CHECK(kitty_pool_release(&pool, stale.data(), max_pages) == KITTY_ERR_INVALID_ARG);
  CHECK(pool.n_free == n_pages && stale[0] == 5);
}

int main() {
  CHECK(kitty_abi_version() == KITTY_ABI_VERSION);
  config_validation();
  workspace_and_plan();
  entry_validation();
  pool_walk();
  std::printf("ok %ld\n", g_checks);
  return 0;
}
