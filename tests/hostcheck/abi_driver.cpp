// Drives every entry point of the WildCat C ABI on the host, for a CPU build under
// AddressSanitizer and UndefinedBehaviorSanitizer with the kernel launchers stubbed out
// (stub_launch.cpp): valid problems on every dispatch path (resident, streaming, block pivots,
// bins with union and per-bin weights, key centring, the cache calls) must return WC_OK with
// every workspace pointer inside the workspace; invalid arguments must return their status
// before any launch; sizes whose workspace would overflow must be refused.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "../../include/wc.h"

extern "C" void wc_hostcheck_set_ws(const void* ws, size_t bytes);
extern "C" long wc_hostcheck_calls(void);

namespace {

int g_fail = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

// A fake device address that converts to any pointer type (never dereferenced: the launchers
// are stubs).
struct Ptr {
  uintptr_t v;
  template <typename T>
  operator T*() const { return reinterpret_cast<T*>(v); }
};
// Caller buffers: distinct 16-byte aligned addresses far below the workspace window.
Ptr buf(int k) { return Ptr{uintptr_t(0x100000000000ull) + uintptr_t(k) * 0x1000000000ull}; }
const Ptr kWs{uintptr_t(0x700000000000ull)};

wc_problem P(int H, int n, int m, int d, int dv, int r, int dtype, int bins = 1, int options = 0, int pb = 1) {
  wc_problem p{};
  p.heads = H; p.n = n; p.m = m; p.d = d; p.dv = dv; p.r = r; p.dtype = dtype;
  p.bins = bins; p.options = options; p.pivot_block = pb;
  return p;
}

void run_valid(const wc_problem& p) {
  size_t ws = 0;
  EXPECT(wc_workspace_bytes(&p, &ws) == WC_OK);
  wc_hostcheck_set_ws((void*)kWs, ws);
  const long before = wc_hostcheck_calls();
  EXPECT(wc_forward(&p, buf(1), buf(2), buf(3), nullptr, 7, buf(4), buf(5), buf(6), buf(7), kWs, ws, nullptr) == WC_OK);
  EXPECT(wc_forward(&p, buf(1), buf(2), buf(3), buf(8), 7, buf(4), nullptr, buf(6), buf(7), kWs, ws, nullptr) == WC_OK);
  if (p.heads > 0) EXPECT(wc_hostcheck_calls() > before);
  // the same call with one byte less of workspace is refused before any launch
  if (ws > 0) {
    const long n0 = wc_hostcheck_calls();
    EXPECT(wc_forward(&p, buf(1), buf(2), buf(3), nullptr, 7, buf(4), buf(5), buf(6), buf(7), kWs, ws - 1, nullptr) ==
           WC_ERR_WORKSPACE);
    EXPECT(wc_hostcheck_calls() == n0);
  }
  if (p.bins <= 1 && !(p.options & WC_OPT_CENTER_KEYS)) {
    EXPECT(wc_rpcholesky(&p, buf(2), nullptr, 1, buf(5), buf(9), buf(10), buf(11), buf(6), buf(7), kWs, ws, nullptr) == WC_OK);
    if (p.pivot_block <= 1) {
      EXPECT(wc_weights(&p, buf(3), buf(5), buf(6), buf(9), buf(12), kWs, ws, nullptr) == WC_OK);
      EXPECT(wc_attend(&p, buf(1), buf(2), buf(5), buf(6), buf(12), buf(4), buf(7), kWs, ws, nullptr) == WC_OK);
    }
    // weights from the keys: their own workspace size, refused one byte short
    size_t kws = 0;
    EXPECT(wc_weights_keys_workspace_bytes(&p, &kws) == WC_OK);
    wc_hostcheck_set_ws((void*)kWs, kws);
    EXPECT(wc_weights_keys(&p, buf(2), buf(3), buf(5), buf(6), buf(12), buf(7), kWs, kws, nullptr) == WC_OK);
    if (kws > 0) {
      const long n0 = wc_hostcheck_calls();
      EXPECT(wc_weights_keys(&p, buf(2), buf(3), buf(5), buf(6), buf(12), buf(7), kWs, kws - 1, nullptr) == WC_ERR_WORKSPACE);
      EXPECT(wc_weights_keys(&p, buf(2), nullptr, buf(5), buf(6), buf(12), buf(7), kWs, kws, nullptr) == WC_ERR_INVALID_ARG);
      EXPECT(wc_hostcheck_calls() == n0);
    }
  } else {
    size_t kws = 1234;
    EXPECT(wc_weights_keys_workspace_bytes(&p, &kws) == WC_ERR_UNSUPPORTED && kws == 1234);
  }
}

void run_cache(const wc_problem& p, int capacity) {
  if (p.options & WC_OPT_CENTER_KEYS) return;
  size_t ws = 0, cb = 0, dws = 0;
  EXPECT(wc_workspace_bytes(&p, &ws) == WC_OK);
  EXPECT(wc_cache_bytes(&p, capacity, &cb) == WC_OK);
  wc_hostcheck_set_ws((void*)kWs, ws);
  EXPECT(wc_compress(&p, buf(2), buf(3), nullptr, 3, buf(13), capacity, buf(5), buf(6), buf(7), kWs, ws, nullptr) == WC_OK);
  EXPECT(wc_cache_append(&p, buf(2), buf(3), 1, p.r, buf(13), capacity, nullptr) == (p.r < capacity ? WC_OK : WC_ERR_INVALID_ARG));
  EXPECT(wc_decode_workspace_bytes(&p, p.r, &dws) == WC_OK);
  wc_hostcheck_set_ws((void*)kWs, dws);
  if (p.m > 0) EXPECT(wc_decode(&p, buf(1), buf(13), capacity, p.r, buf(4), buf(7), kWs, dws, nullptr) == WC_OK);
}

}  // namespace

int main() {
  EXPECT(wc_abi_version() == WC_ABI_VERSION);
  for (int s = 0; s < 8; ++s) EXPECT(wc_status_string((wc_status)s) != nullptr);
  // every dispatch path
  const wc_problem valid[] = {
      P(768, 197, 197, 64, 64, 32, WC_BF16),             // resident
      P(1, 1024, 1024, 64, 64, 32, WC_F32),              // streaming, fp32
      P(32, 4096, 4096, 64, 64, 256, WC_BF16),           // streaming, blocked solve
      P(3, 3001, 77, 128, 64, 33, WC_F32),               // ragged rows
      P(2, 8192, 300, 128, 128, 4096, WC_BF16),          // largest coreset
      P(2, 4096, 64, 128, 128, 256, WC_BF16, 1, 0, 64),  // block pivots
      P(2, 4096, 64, 64, 128, 256, WC_BF16, 16),         // bins, union weights
      P(2, 4096, 64, 64, 64, 256, WC_F32, 8, WC_OPT_BIN_WEIGHTS),
      P(2, 4096, 64, 128, 128, 256, WC_BF16, 8, 0, 32),  // bins with block pivots
      P(2, 2048, 50, 64, 64, 64, WC_BF16, 1, WC_OPT_CENTER_KEYS),
      P(2, 2048, 50, 64, 64, 64, WC_F32, 4, WC_OPT_CENTER_KEYS),
      P(1, 5, 3, 64, 64, 5, WC_BF16),                    // r = n, tiny head
      P(4, 300, 0, 64, 64, 16, WC_F32),                  // no queries
      P(0, 100, 10, 64, 64, 10, WC_BF16),                // no heads
  };
  for (const wc_problem& p : valid) {
    run_valid(p);
    run_cache(p, p.r + 40);
  }
  // invalid arguments: the documented status, no launch
  {
    const wc_problem p = P(2, 1000, 100, 64, 64, 32, WC_BF16);
    size_t ws = 0;
    EXPECT(wc_workspace_bytes(&p, &ws) == WC_OK);
    wc_hostcheck_set_ws((void*)kWs, ws);
    const long n0 = wc_hostcheck_calls();
    const Ptr odd{buf(2).v + 4};
    EXPECT(wc_forward(nullptr, buf(1), buf(2), buf(3), nullptr, 1, buf(4), nullptr, buf(6), buf(7), kWs, ws, nullptr) == WC_ERR_INVALID_ARG);
    EXPECT(wc_forward(&p, buf(1), nullptr, buf(3), nullptr, 1, buf(4), nullptr, buf(6), buf(7), kWs, ws, nullptr) == WC_ERR_INVALID_ARG);
    EXPECT(wc_forward(&p, buf(1), odd, buf(3), nullptr, 1, buf(4), nullptr, buf(6), buf(7), kWs, ws, nullptr) == WC_ERR_INVALID_ARG);
    EXPECT(wc_forward(&p, nullptr, buf(2), buf(3), nullptr, 1, buf(4), nullptr, buf(6), buf(7), kWs, ws, nullptr) == WC_ERR_INVALID_ARG);
    EXPECT(wc_forward(&p, buf(1), buf(2), buf(3), nullptr, 1, buf(4), nullptr, buf(6), buf(7), nullptr, ws, nullptr) == WC_ERR_WORKSPACE);
    EXPECT(wc_rpcholesky(&p, buf(2), odd, 1, buf(5), buf(9), nullptr, nullptr, buf(6), buf(7), kWs, ws, nullptr) == WC_ERR_INVALID_ARG);
    EXPECT(wc_decode(&p, buf(1), buf(13), 10, 11, buf(4), buf(7), kWs, ws, nullptr) == WC_ERR_INVALID_ARG);
    EXPECT(wc_cache_append(&p, buf(2), buf(3), 5, 8, buf(13), 12, nullptr) == WC_ERR_INVALID_ARG);
    const wc_problem bad[] = {
        P(1, 10, 10, 64, 64, 11, WC_BF16), P(1, 10, 10, 64, 64, 0, WC_BF16), P(-1, 10, 10, 64, 64, 5, WC_BF16),
        P(1, 100, 10, 32, 64, 5, WC_BF16), P(1, 100, 10, 64, 96, 5, WC_BF16), P(1, 100, 10, 64, 64, 5, 7),
        P(1, 10000, 10, 64, 64, 4097, WC_BF16), P(2, 4004, 64, 64, 64, 256, WC_BF16, 16),
        P(2, 4096, 64, 64, 64, 256, WC_BF16, 1, 4), P(2, 4096, 64, 64, 64, 250, WC_BF16, 1, 0, 64),
        P(1, 5000000, 10, 64, 64, 5, WC_BF16),
        // workspaces that would not fit in 64 bits (or in any device): refused
        P(2147483647, 4194304, 4194304, 128, 128, 4096, WC_F32), P(1 << 30, 4194304, 1, 128, 128, 4096, WC_BF16),
        P(1 << 20, 1 << 22, 1 << 22, 128, 128, 64, WC_BF16, 64),
    };
    for (const wc_problem& b : bad) {
      size_t x = 1234;
      const wc_status st = wc_workspace_bytes(&b, &x);
      EXPECT(st != WC_OK && x == 1234);
      EXPECT(wc_forward(&b, buf(1), buf(2), buf(3), nullptr, 1, buf(4), nullptr, buf(6), buf(7), kWs, ~size_t(0), nullptr) == st);
    }
    EXPECT(wc_hostcheck_calls() == n0);
  }
  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("hostcheck ok: %ld launches checked\n", wc_hostcheck_calls());
  return 0;
}
