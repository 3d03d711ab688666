// Host-side checks of the C2KV C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitized.py
// builds and runs it).  It drives every entry point's argument validation,
// size queries and host-side planning (tables, split plans, launch chunks)
// with ragged and extreme inputs.  Device pointers are fake, aligned
// addresses: the calls either fail validation before any HIP call or, on a
// machine without a GPU, fail at the first HIP call.  When a GPU is present
// only the host-only closed forms run: no entry point that could launch work
// is ever called with the fake addresses there.
//
// Prints one line per failed expectation and "checks passed: N" at the end;
// exits non-zero on any failure.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "c2kv.h"

namespace {

int g_checks = 0, g_fail = 0;

void expect(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    ++g_fail;
    std::printf("FAILED line %d: %s (last error: %s)\n", line, what, c2kv_last_error());
  }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

void* const FAKE = reinterpret_cast<void*>(uintptr_t{0x10000});
void* const FAKE2 = reinterpret_cast<void*>(uintptr_t{0x20000});
constexpr size_t BIG = size_t{1} << 40;

bool is_err(c2kv_status s) { return s != C2KV_OK; }

// ---------------------------------------------------------- closed forms
void closed_forms() {
  for (int32_t k = 1; k <= 17; ++k)
    for (int32_t n = 0; n <= 300; ++n) {
      const int32_t m = c2kv_num_slots(n, k);
      EXPECT(m == (n + k - 1) / k);
      for (int32_t j = 0; j < m; ++j) {
        const int32_t p = c2kv_slot_position(n, k, j);
        EXPECT(p == std::min(j * k + k - 1, n - 1));
      }
      EXPECT(c2kv_slot_position(n, k, m) == -1);
      EXPECT(c2kv_slot_position(n, k, -1) == -1);
    }
  // extremes: no signed overflow inside the library
  const int32_t big = INT32_MAX;
  for (int32_t k : {1, 2, 7, 1 << 20, big}) {
    const int32_t m = c2kv_num_slots(big, k);
    EXPECT(m >= 1);
    EXPECT(c2kv_slot_position(big, k, m - 1) == big - 1);
    EXPECT(c2kv_slot_position(big, k, 0) == std::min<int64_t>(int64_t{k} - 1, big - 1));
  }
  EXPECT(c2kv_num_slots(-1, 4) == -1);
  EXPECT(c2kv_num_slots(4, 0) == -1);
  float f[64];
  EXPECT(c2kv_rope_inv_freq(128, 5e5f, f) == C2KV_OK);
  EXPECT(f[0] == 1.0f && f[63] > 0.f && f[63] < 1e-4f);
  EXPECT(c2kv_rope_inv_freq(97, 5e5f, f) != C2KV_OK);
  EXPECT(c2kv_rope_inv_freq(1024, 5e5f, f) != C2KV_OK);
  EXPECT(c2kv_rope_inv_freq(64, NAN, f) != C2KV_OK);
  EXPECT(c2kv_rope_inv_freq(64, 1e4f, nullptr) != C2KV_OK);
  for (int s = -1; s <= 6; ++s) EXPECT(c2kv_status_string(static_cast<c2kv_status>(s)) != nullptr);
  EXPECT(std::strlen(c2kv_version()) > 0);
}

// ------------------------------------------------------------ extraction
c2kv_status extract(const std::vector<int32_t>& lens, int32_t k, int32_t sink, int32_t hq, int32_t hkv, int32_t d,
                    c2kv_dtype dt, void* ws, size_t wsb, uint32_t flags = 0, float theta = 1e4f) {
  return c2kv_extract_attn_ex(FAKE, FAKE, FAKE, FAKE2, nullptr, lens.data(), (int32_t)lens.size(), k, sink, hq, hkv,
                              d, theta, dt, flags, ws, wsb, nullptr);
}

void extraction() {
  std::vector<int32_t> ragged;
  for (int i = 0; i < 200; ++i) ragged.push_back(1 + (i * 977) % 5000);
  for (int32_t k : {1, 3, 4, 16})
    for (c2kv_dtype dt : {C2KV_BF16, C2KV_F32}) {
      const size_t ws = c2kv_workspace_size_extract(ragged.data(), (int32_t)ragged.size(), k, 8, 128, dt);
      EXPECT(ws > 0);
      EXPECT(extract(ragged, k, k, 32, 8, 128, dt, FAKE, ws - 1) == C2KV_ERR_WORKSPACE);
      {
        EXPECT(extract(ragged, k, k, 32, 8, 128, dt, FAKE, ws) == C2KV_ERR_HIP);
        EXPECT(extract(ragged, k, 0, 40, 8, 128, dt, FAKE, ws, C2KV_EXTRACT_ANCHOR) == C2KV_ERR_HIP);
      }
    }
  const std::vector<int32_t> two = {16, 9};
  EXPECT(extract(two, 4, 4, 6, 4, 128, C2KV_BF16, FAKE, BIG) == C2KV_ERR_INVALID_ARG);
  EXPECT(extract(two, 4, 4, 34, 2, 128, C2KV_BF16, FAKE, BIG) == C2KV_ERR_UNSUPPORTED);
  EXPECT(extract(two, 4, 4, 4, 2, 96, C2KV_BF16, FAKE, BIG) == C2KV_ERR_UNSUPPORTED);
  EXPECT(extract(two, 0, 4, 4, 2, 128, C2KV_BF16, FAKE, BIG) == C2KV_ERR_INVALID_ARG);
  EXPECT(extract(two, 4, -1, 4, 2, 128, C2KV_BF16, FAKE, BIG) == C2KV_ERR_INVALID_ARG);
  EXPECT(extract(two, 4, 4, 4, 2, 128, C2KV_BF16, FAKE, BIG, 8) == C2KV_ERR_INVALID_ARG);
  EXPECT(extract(two, 4, 4, 4, 2, 128, C2KV_BF16, FAKE, BIG, 0, NAN) == C2KV_ERR_INVALID_ARG);
  EXPECT(extract({16, 0}, 4, 4, 4, 2, 128, C2KV_BF16, FAKE, BIG) == C2KV_ERR_INVALID_ARG);
  EXPECT(extract({1 << 25}, 4, 4, 4, 2, 128, C2KV_BF16, FAKE, BIG) == C2KV_ERR_CAPACITY);
  EXPECT(extract({INT32_MAX, INT32_MAX}, 1, 1, 4, 2, 128, C2KV_BF16, FAKE, BIG) == C2KV_ERR_CAPACITY);
  EXPECT(c2kv_workspace_size_extract(two.data(), 2, 0, 8, 128, C2KV_BF16) == 0);
  EXPECT(c2kv_workspace_size_extract(nullptr, 2, 4, 8, 128, C2KV_BF16) == 0);
  const std::vector<int32_t> huge = {INT32_MAX, INT32_MAX, INT32_MAX};
  EXPECT(c2kv_workspace_size_extract(huge.data(), 3, 1, 8, 128, C2KV_F32) == 0 ||
         c2kv_workspace_size_extract(huge.data(), 3, 1, 8, 128, C2KV_F32) > (size_t{1} << 36));

  // the whole layer
  c2kv_layer_weights w{FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE};
  const size_t lws = c2kv_workspace_size_extract_layer(ragged.data(), 64, 4, 4096, 32, 8, 128, 14336, C2KV_BF16);
  EXPECT(lws > 0);
  auto layer = [&](int32_t dm, int32_t ffn, size_t wsb, const c2kv_layer_weights* wp) {
    return c2kv_extract_layer(FAKE, FAKE2, wp, FAKE, FAKE, ragged.data(), 64, 4, 4, dm, 32, 8, 128, ffn, 5e5f, 1e-5f,
                              C2KV_BF16, FAKE, wsb, nullptr);
  };
  EXPECT(layer(4000, 14336, BIG, &w) == C2KV_ERR_UNSUPPORTED);
  EXPECT(layer(4096, 14336, lws - 1, &w) == C2KV_ERR_WORKSPACE);
  EXPECT(layer(4096, 14336, BIG, nullptr) == C2KV_ERR_INVALID_ARG);
  EXPECT(layer(4096, 14336, lws, &w) == C2KV_ERR_HIP);
}

// ----------------------------------------------------------- composition
struct ComposeCase {
  std::vector<c2kv_segment> segs;
  std::vector<int32_t> ptr{0};
  std::vector<int32_t> base;
  int64_t cap = 0;
};

c2kv_status compose(const ComposeCase& c, int32_t k, int32_t hkv, int32_t d, bool staged = false,
                    size_t wsb = 0) {
  const int32_t R = (int32_t)c.ptr.size() - 1;
  std::vector<int32_t> lens(R + 1, -7), nxt(R + 1, -7);
  const c2kv_status s =
      staged ? c2kv_compose_staged(c.segs.data(), (int32_t)c.segs.size(), c.ptr.data(), R,
                                   c.base.empty() ? nullptr : c.base.data(), k, hkv, d, 1e6f, FAKE, FAKE2, c.cap,
                                   nullptr, lens.data(), nxt.data(), C2KV_BF16, FAKE, wsb, nullptr)
             : c2kv_compose(c.segs.data(), (int32_t)c.segs.size(), c.ptr.data(), R,
                            c.base.empty() ? nullptr : c.base.data(), k, hkv, d, 1e6f, FAKE, FAKE2, c.cap,
                            nullptr, lens.data(), nxt.data(), C2KV_BF16, nullptr, 0, nullptr);
  // host outputs never written past num_reqs
  EXPECT(lens[R] == -7 && nxt[R] == -7);
  return s;
}

void composition() {
  // more distinct documents, occurrences and requests than one launch holds
  ComposeCase big;
  int32_t maxrows = 0;
  for (int r = 0; r < 70; ++r) {
    int32_t rows = 0;
    for (int t = 0; t < 16; ++t) {
      const int doc = (r * 7 + t * 3) % 80;
      const int32_t n = 37 + 61 * doc;
      c2kv_segment s{reinterpret_cast<const char*>(FAKE) + 4096 * doc,
                     reinterpret_cast<const char*>(FAKE2) + 4096 * doc, 256, n, t % 5 == 4 ? 2 : 0};
      big.segs.push_back(s);
      rows += c2kv_num_slots(n, 4);
    }
    big.ptr.push_back((int32_t)big.segs.size());
    big.base.push_back(r * 11);
    maxrows = std::max(maxrows, rows);
  }
  big.cap = maxrows;
  EXPECT(compose(big, 4, 2, 128) == C2KV_ERR_HIP);
  ComposeCase tight = big;
  tight.cap = maxrows - 1;
  EXPECT(compose(tight, 4, 2, 128) == C2KV_ERR_CAPACITY);
  ComposeCase bad = big;
  bad.segs[5].flags = 4;
  EXPECT(compose(bad, 4, 2, 128) == C2KV_ERR_INVALID_ARG);
  bad = big;
  bad.segs[700].doc_len = 0;
  EXPECT(compose(bad, 4, 2, 128) == C2KV_ERR_INVALID_ARG);
  bad = big;
  bad.segs[3].row_stride = 100;
  EXPECT(compose(bad, 4, 2, 128) == C2KV_ERR_INVALID_ARG);
  bad = big;
  bad.ptr.back() -= 1;   // the request table does not cover every segment
  EXPECT(compose(bad, 4, 2, 128) == C2KV_ERR_INVALID_ARG);
  bad = big;
  bad.ptr[10] = bad.ptr[9] - 1;   // not monotone
  EXPECT(compose(bad, 4, 2, 128) == C2KV_ERR_INVALID_ARG);
  bad = big;
  bad.base[69] = (1 << 24) - 10;
  EXPECT(compose(bad, 4, 2, 128) == C2KV_ERR_CAPACITY);
  EXPECT(compose(big, 0, 2, 128) == C2KV_ERR_INVALID_ARG);
  EXPECT(compose(big, 4, 2, 96) == C2KV_ERR_UNSUPPORTED || compose(big, 4, 2, 96) == C2KV_ERR_INVALID_ARG);
  EXPECT(c2kv_workspace_size_compose(100) == 0);
  // staged: the fake addresses are not page-locked host memory
  EXPECT(c2kv_workspace_size_compose_staged(big.segs.data(), (int32_t)big.segs.size(), 4, 2, 128, C2KV_BF16) > 0);
  EXPECT(c2kv_workspace_size_compose_staged(big.segs.data(), (int32_t)big.segs.size(), 0, 2, 128, C2KV_BF16) == 0);
  EXPECT(is_err(compose(big, 4, 2, 128, true, BIG)));
  const void* dp = nullptr;
  std::vector<char> pageable(4096);
  EXPECT(c2kv_host_device_ptr(pageable.data(), pageable.size(), &dp) == C2KV_ERR_INVALID_ARG);
  EXPECT(c2kv_host_device_ptr(nullptr, 16, &dp) == C2KV_ERR_INVALID_ARG);
  EXPECT(c2kv_host_device_ptr(reinterpret_cast<void*>(~uintptr_t{0} - 15), 64, &dp) == C2KV_ERR_INVALID_ARG);
}

// ------------------------------------------------- attention over the cache
void cache_attention() {
  std::vector<int32_t> lens, pos;
  for (int r = 0; r < 150; ++r) {
    lens.push_back(r % 13 == 0 ? 0 : 1 + (r * 2654435761u) % 40000);
    pos.push_back(lens.back() * 4 + 17);
  }
  const int64_t cap = 40100;
  for (c2kv_dtype dt : {C2KV_BF16, C2KV_F32})
    for (int32_t hq : {8, 28, 32}) {
      const int32_t hkv = hq == 28 ? 4 : 8;
      const size_t dws = c2kv_workspace_size_decode(lens.data(), 150, hq, hkv, 128, dt);
      EXPECT(c2kv_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, cap, lens.data(), pos.data(), 150, hq, hkv, 128, 1e6f,
                              FAKE2, nullptr, dt, FAKE, dws == 0 ? 0 : dws - 1, nullptr) ==
             (dws == 0 ? C2KV_OK : C2KV_ERR_WORKSPACE));
      for (int32_t tq : {1, 7, 64}) {
        const size_t pws = c2kv_workspace_size_prefill(lens.data(), 150, tq, hq, hkv, 128, dt);
        EXPECT(pws > 0);
        // many requests: the plan may need no split partials at all
        const c2kv_status s0 = c2kv_attn_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, cap, lens.data(), pos.data(), 150, tq,
                                                 hq, hkv, 128, 1e6f, FAKE2, nullptr, dt, FAKE, 0, nullptr);
        EXPECT(s0 == C2KV_ERR_WORKSPACE || s0 == C2KV_ERR_HIP);
        // one long request is split, and its partials need the workspace
        const size_t pws1 = c2kv_workspace_size_prefill(lens.data() + 1, 1, tq, hq, hkv, 128, dt);
        EXPECT(c2kv_attn_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, cap, lens.data() + 1, pos.data() + 1, 1, tq, hq, hkv,
                                 128, 1e6f, FAKE2, nullptr, dt, FAKE, pws1 - 1, nullptr) == C2KV_ERR_WORKSPACE);
        EXPECT(c2kv_attn_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, cap, lens.data(), pos.data(), 150, tq, hq, hkv,
                                   128, 1e6f, FAKE2, nullptr, dt, FAKE, pws, nullptr) == C2KV_ERR_HIP);
      }
      {
        EXPECT(c2kv_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, cap, lens.data(), pos.data(), 150, hq, hkv, 128, 1e6f,
                                FAKE2, nullptr, dt, FAKE, BIG, nullptr) == C2KV_ERR_HIP);
        EXPECT(c2kv_attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, cap, lens.data(), pos.data(), 150, hq, hkv,
                                        128, 1e6f, FAKE2, nullptr, dt, nullptr) == C2KV_ERR_HIP);
      }
    }
  std::vector<int32_t> full = {40100}, p0 = {0};
  EXPECT(c2kv_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, cap, full.data(), p0.data(), 1, 8, 2, 128, 1e6f, FAKE2,
                          nullptr, C2KV_BF16, FAKE, BIG, nullptr) == C2KV_ERR_CAPACITY);
  std::vector<int32_t> neg = {-1};
  EXPECT(c2kv_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, cap, neg.data(), p0.data(), 1, 8, 2, 128, 1e6f, FAKE2,
                          nullptr, C2KV_BF16, FAKE, BIG, nullptr) == C2KV_ERR_INVALID_ARG);
  EXPECT(c2kv_attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, cap, neg.data(), p0.data(), 1, 8, 2, 128, 1e6f,
                                  FAKE2, nullptr, C2KV_BF16, nullptr) == C2KV_ERR_INVALID_ARG);
  // (cap + 256) rows of one KV head must stay below 2 GiB
  std::vector<int32_t> one = {5};
  EXPECT(c2kv_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, int64_t{1} << 23, one.data(), p0.data(), 1, 8, 2, 128, 1e6f,
                          FAKE2, nullptr, C2KV_F32, FAKE, BIG, nullptr) == C2KV_ERR_CAPACITY);
  EXPECT(c2kv_workspace_init(FAKE, 6, nullptr) == C2KV_ERR_INVALID_ARG);
  EXPECT(c2kv_workspace_init(FAKE, 4096, nullptr) == C2KV_ERR_HIP);
}

// ------------------------------------------------------------ test support
void test_support() {
  uint64_t counts[5];
  std::vector<int32_t> lens = {12, 100, 3, 4097};
  const size_t mws = c2kv_workspace_size_mask_cells();
  EXPECT(c2kv_mask_cells(lens.data(), 4, 4, 4, nullptr, FAKE, mws, nullptr) == C2KV_ERR_INVALID_ARG);
  EXPECT(c2kv_mask_cells(lens.data(), 4, 4, 4, counts, FAKE, mws - 1, nullptr) == C2KV_ERR_WORKSPACE);
  EXPECT(c2kv_mask_cells_ex(lens.data(), 4, 4, 4, 2, counts, FAKE, mws, nullptr) == C2KV_ERR_INVALID_ARG);
  const size_t tws = c2kv_workspace_size_tile_schedule();
  int64_t cnt = -1;
  EXPECT(c2kv_tile_schedule(lens.data(), 4, 4, 4, 8, 2, 0, nullptr, 0, nullptr, FAKE, tws, nullptr) ==
         C2KV_ERR_INVALID_ARG);
  EXPECT(c2kv_tile_schedule(lens.data(), 4, 4, 4, 34, 2, 0, nullptr, 0, &cnt, FAKE, tws, nullptr) ==
         C2KV_ERR_UNSUPPORTED);
  EXPECT(c2kv_tile_schedule(lens.data(), 4, 4, 4, 8, 2, 0, nullptr, 5, &cnt, FAKE, tws, nullptr) ==
         C2KV_ERR_INVALID_ARG);
  {
    EXPECT(c2kv_mask_cells(lens.data(), 4, 4, 4, counts, FAKE, mws, nullptr) == C2KV_ERR_HIP);
    EXPECT(c2kv_tile_schedule(lens.data(), 4, 4, 4, 8, 2, C2KV_EXTRACT_ANCHOR, nullptr, 0, &cnt, FAKE, tws,
                              nullptr) == C2KV_ERR_HIP);
  }
}

}  // namespace

int main() {
  int ndev = 0;
  const bool no_gpu = hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0;
  (void)hipGetLastError();
  std::printf("devices: %d (%s)\n", ndev, no_gpu ? "planning paths run up to the first HIP call" :
                                                   "closed forms only");
  closed_forms();
  if (no_gpu) {
    extraction();
    composition();
    cache_attention();
    test_support();
  }
  std::printf("checks passed: %d of %d\n", g_checks - g_fail, g_checks);
  return g_fail == 0 ? 0 : 1;
}
