// Host-only stand-ins for the kernel launchers of the WildCat library, for a CPU build of the
// C ABI (wc_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.  No device memory is
// touched: every launcher checks that each workspace pointer it is handed lies inside the
// workspace the caller registered (wc_hostcheck_set_ws), counts the call and returns success.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "../../coreset_head_rpcholesky_amd/csrc/wc_kernels.h"

namespace {
uintptr_t g_ws = 0;
size_t g_ws_bytes = 0;
long g_calls = 0;

// A pointer inside the workspace window [ws, ws + 2^40) must fall in [ws, ws + ws_bytes) and be
// 16-byte aligned; pointers elsewhere are caller buffers and are not checked here.
void check(const void* p, const char* what) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(p);
  if (!p || g_ws == 0 || x < g_ws || x >= g_ws + (uintptr_t(1) << 40)) return;
  if (x >= g_ws + g_ws_bytes || (x & 15u)) {
    std::fprintf(stderr, "workspace pointer %s at offset %zu outside %zu bytes or misaligned\n", what,
                 (size_t)(x - g_ws), g_ws_bytes);
    std::abort();
  }
}
#define CHK(field) check(reinterpret_cast<const void*>(a.field), #field)
}  // namespace

extern "C" void wc_hostcheck_set_ws(const void* ws, size_t bytes) {
  g_ws = reinterpret_cast<uintptr_t>(ws);
  g_ws_bytes = bytes;
}
extern "C" long wc_hostcheck_calls(void) { return g_calls; }

namespace wc {

static hipError_t resident(const ResidentArgs& a) {
  CHK(Q); CHK(K); CHK(V); CHK(pivots); CHK(F); CHK(diag); CHK(trace); CHK(rank); CHK(flags); CHK(W); CHK(O);
  ++g_calls;
  return hipSuccess;
}
hipError_t launch_resident_64_64(const ResidentArgs& a, int, hipStream_t) { return resident(a); }
hipError_t launch_resident_64_128(const ResidentArgs& a, int, hipStream_t) { return resident(a); }
hipError_t launch_resident_128_64(const ResidentArgs& a, int, hipStream_t) { return resident(a); }
hipError_t launch_resident_128_128(const ResidentArgs& a, int, hipStream_t) { return resident(a); }

static void stream_args(const StreamRpcArgs& a) {
  CHK(K); CHK(u_forced); CHK(uniforms); CHK(F); CHK(diag0); CHK(diag1); CHK(part0); CHK(part1);
  CHK(pivots); CHK(trace); CHK(rank); CHK(flags); CHK(diag_out);
  if (a.nblk < 1 || a.nblk > 4096 || (a.rows != 256 && a.rows != 1024)) {
    std::fprintf(stderr, "pivot loop launched with rows %d, nblk %d\n", a.rows, a.nblk);
    std::abort();
  }
}
hipError_t launch_rpc_stream(const StreamRpcArgs& a, hipStream_t) {
  stream_args(a);
  ++g_calls;
  return hipSuccess;
}
hipError_t launch_rpc_block(const BlockRpcArgs& a, hipStream_t) {
  stream_args(a.s);
  CHK(cand); CHK(slot); CHK(G); CHK(M); CHK(rounds); CHK(FS);
  ++g_calls;
  return hipSuccess;
}
hipError_t launch_weights(const WeightsArgs& a, hipStream_t) {
  CHK(V); CHK(F); CHK(pivots); CHK(rank); CHK(L); CHK(Xpart); CHK(X); CHK(W); CHK(Minv);
  ++g_calls;
  return hipSuccess;
}
hipError_t launch_bins_combine(const BinsArgs& a, hipStream_t) {
  CHK(piv_sub); CHK(rank_sub); CHK(flags_sub); CHK(pivots); CHK(rank); CHK(flags); CHK(rank_slots);
  ++g_calls;
  return hipSuccess;
}
// split: the launch runs the attention proper, whose coreset split must be set
static hipError_t attend(const AttendArgs& a, bool split) {
  CHK(Q); CHK(K); CHK(V); CHK(pivots); CHK(rank); CHK(W); CHK(KSh); CHK(KSl); CHK(Wph); CHK(Wpl);
  CHK(Wden); CHK(Wdh); CHK(Ypart); CHK(O); CHK(flags); CHK(Yout);
  if (split && (a.nsplit < 1 || (a.nsplit > 1 && !a.Ypart))) {
    std::fprintf(stderr, "attention launched with nsplit %d\n", a.nsplit);
    std::abort();
  }
  ++g_calls;
  return hipSuccess;
}
hipError_t launch_attend(const AttendArgs& a, hipStream_t) { return attend(a, a.m > 0); }
hipError_t launch_attend_all_keys(const AttendArgs& a, hipStream_t) { return attend(a, a.m > 0); }
hipError_t launch_attend_prep(const AttendArgs& a, hipStream_t) { return attend(a, false); }
hipError_t launch_attend_append(const AttendArgs& a, hipStream_t) { return attend(a, false); }
hipError_t launch_attend_core(const AttendArgs& a, hipStream_t) { return attend(a, true); }
hipError_t launch_decode(const AttendArgs& a, hipStream_t) { return attend(a, false); }
hipError_t launch_union_gather(const UnionArgs& a, hipStream_t) {
  CHK(K); CHK(pivots); CHK(Qs); CHK(A); CHK(Hd); CHK(M); CHK(X); CHK(W); CHK(flags);
  ++g_calls;
  return hipSuccess;
}
hipError_t launch_union_solve(const UnionArgs& a, hipStream_t s) { return launch_union_gather(a, s); }
hipError_t launch_union_mask(const int32_t* pivots, const int32_t* rank, int32_t* out, int, int, hipStream_t) {
  check(pivots, "pivots"); check(rank, "rank"); check(out, "out");
  ++g_calls;
  return hipSuccess;
}
hipError_t launch_union_back(const UnionArgs& a, hipStream_t s) { return launch_union_gather(a, s); }
hipError_t launch_center(const CenterArgs& a, hipStream_t) {
  CHK(K); CHK(part); CHK(mean); CHK(Kc);
  ++g_calls;
  return hipSuccess;
}

}  // namespace wc
