// C ABI of the WildCat hot path: argument validation, workspace carving and dispatch.
//
// Every entry point validates on the host before touching HIP; on failure it returns a
// status and enqueues nothing.  Dispatch: heads of at most 256 bf16 keys with r <= 32 run
// the resident kernel (one workgroup per head, the whole forward in one launch); all other
// problems run the streaming pivot loop (one launch per pivot step), the factor-based
// weights and the matrix-core attention.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/wc.h"
#include "wc_host.h"
#include "wc_kernels.h"

namespace {

constexpr int kMaxR = 4096;
constexpr int kMaxBlocks = 4096;  // row blocks of the streaming pivot loop per head

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

wc_status check_problem(const wc_problem* p) {
  if (!p) return WC_ERR_INVALID_ARG;
  if (p->heads < 0 || p->n < 1 || p->m < 0 || p->r < 1) return WC_ERR_INVALID_ARG;
  if (p->r > p->n) return WC_ERR_INVALID_ARG;
  if ((p->d != 64 && p->d != 128) || (p->dv != 64 && p->dv != 128)) return WC_ERR_UNSUPPORTED;
  if (p->dtype != WC_F32 && p->dtype != WC_BF16) return WC_ERR_UNSUPPORTED;
  if (p->r > kMaxR) return WC_ERR_UNSUPPORTED;
  if (p->bins < 0) return WC_ERR_INVALID_ARG;
  if ((uint32_t)p->options & ~(uint32_t)(WC_OPT_BIN_WEIGHTS | WC_OPT_CENTER_KEYS)) return WC_ERR_INVALID_ARG;
  if (p->pivot_block < 0) return WC_ERR_INVALID_ARG;
  if (p->pivot_block > 1) {
    const int B = p->bins > 1 ? p->bins : 1;
    if (p->pivot_block != 16 && p->pivot_block != 32 && p->pivot_block != 64) return WC_ERR_UNSUPPORTED;
    if ((p->r / B) % p->pivot_block != 0) return WC_ERR_UNSUPPORTED;
  }
  if (p->bins > 1 && (p->n % p->bins != 0 || p->r % p->bins != 0)) return WC_ERR_UNSUPPORTED;
  if ((int64_t)p->n > (int64_t)kMaxBlocks * 1024) return WC_ERR_UNSUPPORTED;
  // sizes whose buffers could not exist on any device (and whose workspace arithmetic would
  // leave 64 bits): more than 2^48 elements in one array
  const double rows = (double)p->heads * (p->n > p->m ? p->n : p->m);
  const double width = (double)(p->r > 128 ? p->r : 128) + 1.0;
  if (rows * width > 281474976710656.0) return WC_ERR_UNSUPPORTED;
  return WC_OK;
}

// A required device pointer: non-null and 16-byte aligned.
bool req(const void* ptr) { return ptr != nullptr && aligned16(ptr); }
// An optional device pointer: null, or 16-byte aligned.
bool opt(const void* ptr) { return ptr == nullptr || aligned16(ptr); }

bool resident_ok(const wc_problem& p) {
  return p.dtype == WC_BF16 && p.n <= wc::kResidentRows && p.r <= wc::kResidentR && p.pivot_block <= 1;
}

bool binned(const wc_problem& p) { return p.bins > 1; }
// Weights solve: blocked back substitution over 64-row blocks (one launch per block, all blocks
// of the update in parallel) for large coresets, the one-pass trisolve otherwise.
bool blocked_solve(const wc_problem& p) { return p.r % 64 == 0 && p.r >= 256; }
bool blocked(const wc_problem& p) { return p.pivot_block > 1; }
// Bins go through the per-bin selection, the fold of the pivots and weights over the union.
bool union_path(const wc_problem& p) { return binned(p); }
bool union_weights(const wc_problem& p) { return union_path(p) && !(p.options & WC_OPT_BIN_WEIGHTS); }
bool centred(const wc_problem& p) { return (p.options & WC_OPT_CENTER_KEYS) != 0; }

// The per-bin view of a binned problem: heads * B sub-heads of n/B keys and r/B pivots (a
// problem with one bin is its own view).
wc_problem sub_problem(const wc_problem& p) {
  wc_problem s = p;
  const int B = p.bins > 1 ? p.bins : 1;
  s.heads = p.heads * B;
  s.n = p.n / B;
  s.r = p.r / B;
  s.m = 0;
  s.bins = 1;
  s.options = 0;
  return s;
}

// Coreset split of the attention: when the query tiles alone give too few workgroups, the
// coreset rows (chunks of 64 for bf16, 32 for fp32) are shared out over nsplit workgroups
// whose partial sums are reduced afterwards.
int attend_split(const wc_problem& p, size_t m, size_t coreset_rows) {
  const size_t H = (size_t)p.heads;
  const size_t cw = p.dtype == WC_BF16 ? 64 : 32;
  const size_t qw = p.dtype == WC_BF16 ? 256 : 128;
  const size_t nchk = (size_t)wc::attend_rows((int)coreset_rows) / cw;
  const size_t qtiles = (m + qw - 1) / qw;
  size_t nsplit = 1;
  if (qtiles * H < 512 && qtiles > 0) {
    nsplit = (512 + qtiles * H - 1) / (qtiles * H);
    if (nsplit > nchk) nsplit = nchk;
    const size_t per = (nchk + nsplit - 1) / nsplit;
    nsplit = (nchk + per - 1) / per;
  }
  return (int)nsplit;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  int rows, nblk, nchunk, chunk_rows, nsplit, rp;
  size_t diag0, diag1, part0, part1, unif, F, piv, L, Xpart, X, W, Minv, KSh, KSl, Wph, Wpl, Wden, Wdh, Ypart;
  size_t bcand, bslot, bG, bM, brounds, bFS;  // block pivot selection
  size_t total;
};

// parts: kSelect (pivot loop and weights) and/or kAttend (staged coreset and attention).
constexpr int kSelect = 1, kAttend = 2;

Layout make_layout(const wc_problem& p, int parts = kSelect | kAttend) {
  Layout L{};
  const size_t H = (size_t)p.heads, n = (size_t)p.n, r = (size_t)p.r, m = (size_t)p.m;
  const size_t nc = (size_t)p.dv + 1;
  // pivot loop: 1024 rows per workgroup (4 contiguous rows per thread, 16-byte accesses)
  // when n is a multiple of 4 and that still gives enough workgroups to fill the chip;
  // otherwise 256 rows (one per thread)
  L.rows = (n % 4 == 0 && H * ((n + 1023) / 1024) >= 512) ? 1024 : 256;
  L.nblk = (int)((n + L.rows - 1) / L.rows);
  // weights: key chunks so that (r/256 row groups) x chunks x heads >= 512 workgroups
  const size_t jg = (r + 255) / 256;
  size_t nchunk = (512 + jg * H - 1) / (jg * H);
  const size_t maxchunk = (n + 63) / 64;
  if (nchunk > maxchunk) nchunk = maxchunk;
  if (nchunk < 1) nchunk = 1;
  size_t crow = (n + nchunk - 1) / nchunk;
  crow = (crow + 63) & ~size_t(63);
  L.chunk_rows = (int)crow;
  L.nchunk = (int)((n + crow - 1) / crow);
  L.rp = wc::attend_rows((int)r);
  L.nsplit = attend_split(p, m, r);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  if (parts & kSelect) {
    L.diag0 = take(H * n * 4);
    L.diag1 = take(H * n * 4);
    L.part0 = take(H * L.nblk * 8);
    L.part1 = take(H * L.nblk * 8);
    L.unif = take(H * r * 4 * (blocked(p) ? wc::kBlockDraws : 1));
    L.F = take(H * r * n * 4);
    L.piv = take(H * r * 4);
    L.L = take(H * r * r * 4);
    L.Xpart = take(H * L.nchunk * r * nc * 4);
    L.X = take(H * r * nc * 4);
    L.W = take(H * r * nc * 4);
    L.Minv = blocked_solve(p) ? take(H * r * 64 * 4) : 0;
    if (blocked(p)) {
      const size_t b = (size_t)p.pivot_block;
      L.bcand = take(H * b * 4);
      L.bslot = take(H * b * 4);
      L.bG = take(H * b * n * 4);
      L.bM = take(H * b * b * 4);
      L.brounds = take(H * 4);
      L.bFS = take(H * r * b * 4);
    }
  }
  if (parts & kAttend) {
    const size_t lo = p.dtype == WC_F32 ? 1 : 0;  // lo parts of the bf16 splits: fp32 only
    L.KSh = take(H * L.rp * p.d * 2);
    L.KSl = take(lo * H * L.rp * p.d * 2);
    L.Wph = take(H * p.dv * L.rp * 2);
    L.Wpl = take(lo * H * p.dv * L.rp * 2);
    L.Wden = take(H * L.rp * 4);
    L.Wdh = take(H * L.rp * 2);
    L.Ypart = take(L.nsplit > 1 ? H * L.nsplit * m * nc * 4 : 0);
  }
  L.total = off;
  return L;
}

// Buffers of the union weights W = H_SS^+ H_{S,:} [V, 1] for r slots per head, from `base` on:
// the slots' pivots (a copy masked by rank, for wc_weights_keys), the coreset keys as rows,
// the all-keys pass X = exp(beta K_S K^T) [V, 1] and the blocked solve.
struct UnionLayout {
  int urp, xsplit;
  size_t piv, Qs, A, Hd, M, X, xKSh, xKSl, xWph, xWpl, xWden, xWdh, xYpart, total;
};

UnionLayout make_union_layout(const wc_problem& p, size_t base) {
  UnionLayout U{};
  const size_t H = (size_t)p.heads, r = (size_t)p.r, n = (size_t)p.n, nc = (size_t)p.dv + 1;
  const size_t esz = p.dtype == WC_F32 ? 4 : 2, lo = p.dtype == WC_F32 ? 1 : 0;
  const size_t urp = (r + 63) & ~size_t(63), np = (size_t)wc::attend_rows(p.n);
  size_t off = align_up(base);
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  U.urp = (int)urp;
  U.xsplit = attend_split(p, r, n);
  U.piv = take(H * r * 4);
  U.Qs = take(H * r * p.d * esz);
  U.A = take(H * urp * urp * 4);
  U.Hd = take(H * urp * 4);
  U.M = take(H * urp * 64 * 4);
  U.X = take(H * urp * nc * 4);
  U.xKSh = take(lo * H * np * p.d * 2);   // bf16 keys are read in place by the all-keys pass
  U.xKSl = take(lo * H * np * p.d * 2);
  U.xWph = take(H * p.dv * np * 2);
  U.xWpl = take(lo * H * p.dv * np * 2);
  U.xWden = take(H * np * 4);
  U.xWdh = take(H * np * 2);
  U.xYpart = take(U.xsplit > 1 ? H * U.xsplit * r * nc * 4 : 0);
  U.total = off;
  return U;
}

// Workspace of a binned forward: the per-bin selection and weights (the sub-head layout, whose
// W is the heads' W), the heads' attention buffers, the per-bin outputs, and for the union
// weights the union buffers.
struct BinnedLayout {
  Layout sub, head;
  size_t head_base, piv_sub, rank_sub, flags_sub, rank_slots, piv, total;
  UnionLayout U;
};

BinnedLayout make_binned_layout(const wc_problem& p) {
  BinnedLayout B{};
  wc_problem hp = p;
  hp.bins = 1;
  B.sub = make_layout(sub_problem(p), kSelect);
  B.head = make_layout(hp, kAttend);
  const size_t H = (size_t)p.heads, r = (size_t)p.r;
  size_t off = align_up(B.sub.total);
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  B.head_base = take(B.head.total);
  B.piv_sub = take(H * r * 4);
  B.rank_sub = take(H * p.bins * 4);
  B.flags_sub = take(H * p.bins * 4);
  B.rank_slots = take(H * 4);
  B.piv = take(H * r * 4);
  if (union_weights(p)) {
    B.U = make_union_layout(p, off);
    off = B.U.total;
  }
  B.total = off;
  return B;
}

// Key centring keeps its buffers after everything else: the centred keys, the per-block fp64
// column sums and the mean.
struct CenterLayout {
  size_t Kc, part, mean, total;
};

CenterLayout make_center_layout(const wc_problem& p, size_t base) {
  CenterLayout C{};
  const size_t H = (size_t)p.heads, esz = p.dtype == WC_F32 ? 4 : 2;
  size_t off = align_up(base);
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  C.Kc = take(H * p.n * p.d * esz);
  C.part = take(H * wc::center_blocks(p.n) * p.d * 8);
  C.mean = take(H * p.d * 8);
  C.total = off;
  return C;
}

size_t workspace_total(const wc_problem& p) {
  const size_t base = union_path(p) ? make_binned_layout(p).total : make_layout(p).total;
  return centred(p) ? make_center_layout(p, base).total : base;
}

template <typename Tp>
Tp* at(void* ws, size_t off) { return reinterpret_cast<Tp*>(static_cast<char*>(ws) + off); }

wc_status check_ws(const wc_problem& p, const void* ws, size_t ws_bytes, Layout* lay) {
  *lay = make_layout(p);
  if (!ws || !aligned16(ws) || ws_bytes < lay->total) return WC_ERR_WORKSPACE;
  return WC_OK;
}

float beta_log2e(int d) { return (float)(1.4426950408889634 / std::sqrt((double)d)); }

wc_status dev(hipError_t e) { return e == hipSuccess ? WC_OK : WC_ERR_DEVICE; }

hipError_t run_rpc_stream(const wc_problem& p, const Layout& L, void* ws, const void* K,
                          const float* u_forced, uint64_t seed, int32_t* pivots, float* F,
                          float* diag, double* trace, int32_t* rank, uint32_t* flags,
                          hipStream_t st) {
  wc::StreamRpcArgs a{};
  a.K = K;
  a.bf16 = p.dtype == WC_BF16;
  a.u_forced = u_forced;
  a.seed = seed;
  a.uniforms = u_forced ? const_cast<float*>(u_forced) : at<float>(ws, L.unif);
  a.H = p.heads; a.n = p.n; a.d = p.d; a.r = p.r;
  a.rows = L.rows; a.nblk = L.nblk;
  a.beta_log2e = beta_log2e(p.d);
  a.F = F;
  a.diag0 = at<float>(ws, L.diag0);
  a.diag1 = at<float>(ws, L.diag1);
  a.part0 = at<double>(ws, L.part0);
  a.part1 = at<double>(ws, L.part1);
  a.pivots = pivots; a.trace = trace; a.rank = rank; a.flags = flags; a.diag_out = diag;
  return wc::launch_rpc_stream(a, st);
}

hipError_t run_weights(const wc_problem& p, const Layout& L, void* ws, const void* V,
                       const int32_t* pivots, const int32_t* rank, const float* F, float* W,
                       hipStream_t st, uint32_t* flags = nullptr) {
  wc::WeightsArgs a{};
  a.V = V;
  a.bf16 = p.dtype == WC_BF16;
  a.H = p.heads; a.n = p.n; a.dv = p.dv; a.r = p.r;
  a.F = F; a.pivots = pivots; a.rank = rank;
  a.L = at<float>(ws, L.L);
  a.Xpart = at<float>(ws, L.Xpart);
  a.nchunk = L.nchunk; a.chunk_rows = L.chunk_rows;
  a.X = at<float>(ws, L.X);
  a.W = W;
  a.Minv = blocked_solve(p) ? at<float>(ws, L.Minv) : nullptr;
  a.flags = flags;
  return wc::launch_weights(a, st);
}

hipError_t run_attend(const wc_problem& p, const Layout& L, void* ws, const void* Q,
                      const void* K, const int32_t* pivots, const int32_t* rank,
                      const float* W, void* O, uint32_t* flags, hipStream_t st) {
  wc::AttendArgs a{};
  a.Q = Q; a.K = K;
  a.bf16 = p.dtype == WC_BF16;
  a.H = p.heads; a.n = p.n; a.m = p.m; a.d = p.d; a.dv = p.dv; a.r = p.r;
  a.beta_log2e = beta_log2e(p.d);
  a.pivots = pivots; a.rank = rank; a.W = W;
  a.KSh = at<uint16_t>(ws, L.KSh);
  a.KSl = p.dtype == WC_F32 ? at<uint16_t>(ws, L.KSl) : nullptr;
  a.Wph = at<uint16_t>(ws, L.Wph);
  a.Wpl = p.dtype == WC_F32 ? at<uint16_t>(ws, L.Wpl) : nullptr;
  a.Wden = at<float>(ws, L.Wden);
  a.Wdh = at<uint16_t>(ws, L.Wdh);
  a.Ypart = L.nsplit > 1 ? at<float>(ws, L.Ypart) : nullptr;
  a.nsplit = L.nsplit;
  a.O = O; a.flags = flags;
  return wc::launch_attend(a, st);
}

// Pivot loop for every head of p (resident kernel when it fits, else the streaming loop).
hipError_t run_rpc_block(const wc_problem& p, const Layout& L, void* ws, const void* K,
                         const float* u_forced, uint64_t seed, int32_t* pivots, float* F,
                         float* diag, double* trace, int32_t* rank, uint32_t* flags, hipStream_t st) {
  wc::BlockRpcArgs a{};
  wc::StreamRpcArgs& s = a.s;
  s.K = K;
  s.bf16 = p.dtype == WC_BF16;
  s.u_forced = u_forced;
  s.seed = seed;
  s.uniforms = u_forced ? const_cast<float*>(u_forced) : at<float>(ws, L.unif);
  s.H = p.heads; s.n = p.n; s.d = p.d; s.r = p.r;
  s.rows = L.rows; s.nblk = L.nblk;
  s.beta_log2e = beta_log2e(p.d);
  s.F = F;
  s.diag0 = at<float>(ws, L.diag0);
  s.diag1 = at<float>(ws, L.diag1);
  s.part0 = at<double>(ws, L.part0);
  s.part1 = at<double>(ws, L.part1);
  s.pivots = pivots; s.trace = trace; s.rank = rank; s.flags = flags; s.diag_out = diag;
  a.b = p.pivot_block;
  a.tol = 0x1p-12f;
  a.cand = at<int32_t>(ws, L.bcand);
  a.slot = at<int32_t>(ws, L.bslot);
  a.G = at<float>(ws, L.bG);
  a.M = at<float>(ws, L.bM);
  a.rounds = at<int32_t>(ws, L.brounds);
  a.FS = at<float>(ws, L.bFS);
  return wc::launch_rpc_block(a, st);
}

hipError_t run_select(const wc_problem& p, const Layout& L, void* ws, const void* K,
                      const float* u_forced, uint64_t seed, int32_t* pivots, float* F,
                      int32_t* rank, uint32_t* flags, hipStream_t st) {
  if (blocked(p)) return run_rpc_block(p, L, ws, K, u_forced, seed, pivots, F, nullptr, nullptr, rank, flags, st);
  if (resident_ok(p)) {
    wc::ResidentArgs a{};
    a.K = static_cast<const uint16_t*>(K);
    a.u_forced = u_forced; a.seed = seed;
    a.n = p.n; a.m = 0; a.r = p.r;
    a.beta_log2e = beta_log2e(p.d);
    a.pivots = pivots; a.F = F; a.rank = rank; a.flags = flags;
    return wc::launch_resident(a, p.heads, p.d, p.dv, st);
  }
  return run_rpc_stream(p, L, ws, K, u_forced, seed, pivots, F, nullptr, nullptr, rank, flags, st);
}

// W = H_SS^+ H_{S,:} [V, 1] over the slots `piv` (-1: empty) of every head, into W
// [heads][r][dv+1] (gist.science/de/paper/2602.10056, "Methodik" part 2, with the
// pseudo-inverse taken by the leave-out Cholesky of the union kernels).
hipError_t run_union_weights(const wc_problem& p, const UnionLayout& U, void* ws, const void* K,
                             const void* V, const int32_t* piv, float* W, uint32_t* flags,
                             hipStream_t s) {
  wc::UnionArgs u{};
  u.K = K; u.bf16 = p.dtype == WC_BF16;
  u.H = p.heads; u.n = p.n; u.d = p.d; u.dv = p.dv; u.r = p.r; u.rp = U.urp;
  u.beta = (float)(1.0 / std::sqrt((double)p.d));
  u.tol = 0x1p-12f;
  u.pivots = piv;
  u.Qs = at<void>(ws, U.Qs);
  u.A = at<float>(ws, U.A); u.Hd = at<float>(ws, U.Hd); u.M = at<float>(ws, U.M);
  u.X = at<float>(ws, U.X); u.W = W; u.flags = flags;
  hipError_t e = wc::launch_union_gather(u, s);
  if (e == hipSuccess) {
    // X = exp(beta K_S K^T) [V, 1]: the attention kernels with the coreset keys as queries
    // and every key as a coreset row
    wc::AttendArgs x{};
    x.Q = u.Qs; x.K = K; x.V = V;
    x.bf16 = u.bf16;
    x.H = p.heads; x.n = p.n; x.m = p.r; x.d = p.d; x.dv = p.dv; x.r = p.n;
    x.beta_log2e = beta_log2e(p.d);
    x.KSh = p.dtype == WC_F32 ? at<uint16_t>(ws, U.xKSh) : nullptr;   // bf16: keys read in place
    x.KSl = p.dtype == WC_F32 ? at<uint16_t>(ws, U.xKSl) : nullptr;
    x.Wph = at<uint16_t>(ws, U.xWph);
    x.Wpl = p.dtype == WC_F32 ? at<uint16_t>(ws, U.xWpl) : nullptr;
    x.Wden = at<float>(ws, U.xWden);
    x.Wdh = at<uint16_t>(ws, U.xWdh);
    x.nsplit = U.xsplit;
    x.Ypart = U.xsplit > 1 ? at<float>(ws, U.xYpart) : nullptr;
    x.flags = flags;
    x.Yout = u.X; x.yrows = U.urp;
    e = wc::launch_attend_all_keys(x, s);
  }
  if (e == hipSuccess) e = wc::launch_union_solve(u, s);
  return e;
}

// Divide-and-conquer forward: selection and weights per bin on the sub-head view (the keys,
// values and forced uniforms of bin b of head h are those of sub-head h B + b, contiguous),
// pivots folded back to key indices of the head, then attention over the union.
wc_status forward_binned(const wc_problem& p, const void* Q, const void* K, const void* V,
                         const float* u_forced, uint64_t seed, void* O, int32_t* pivots,
                         int32_t* rank, uint32_t* flags, void* ws, size_t ws_bytes, hipStream_t s) {
  const BinnedLayout B = make_binned_layout(p);
  if (!ws || !aligned16(ws) || ws_bytes < B.total) return WC_ERR_WORKSPACE;
  const wc_problem sp = sub_problem(p);
  int32_t* piv_sub = at<int32_t>(ws, B.piv_sub);
  int32_t* rank_sub = at<int32_t>(ws, B.rank_sub);
  uint32_t* flags_sub = at<uint32_t>(ws, B.flags_sub);
  float* F = at<float>(ws, B.sub.F);
  float* W = at<float>(ws, B.sub.W);
  hipError_t e = run_select(sp, B.sub, ws, K, u_forced, seed, piv_sub, F, rank_sub, flags_sub, s);
  if (e == hipSuccess && !union_weights(p)) e = run_weights(sp, B.sub, ws, V, piv_sub, rank_sub, F, W, s, flags_sub);
  int32_t* piv = pivots ? pivots : at<int32_t>(ws, B.piv);
  int32_t* slots = at<int32_t>(ws, B.rank_slots);
  if (e == hipSuccess) {
    wc::BinsArgs a{};
    a.H = p.heads; a.B = p.bins; a.nb = sp.n; a.rb = sp.r;
    a.piv_sub = piv_sub; a.rank_sub = rank_sub; a.flags_sub = flags_sub;
    a.pivots = piv; a.rank = rank; a.flags = flags; a.rank_slots = slots;
    e = wc::launch_bins_combine(a, s);
  }
  if (e == hipSuccess && union_weights(p)) e = run_union_weights(p, B.U, ws, K, V, piv, W, flags, s);
  wc_problem hp = p;
  hp.bins = 1;
  if (e == hipSuccess && p.m > 0)
    e = run_attend(hp, B.head, static_cast<char*>(ws) + B.head_base, Q, K, piv, slots, W, O, flags, s);
  return dev(e);
}

// Compressed KV cache: per head, capacity rows (rounded up to whole 128-row blocks) in the
// staged layout of the attention kernels (keys tile-major, weights transposed and permuted).
struct CacheLayout {
  int cp;
  size_t KSh, KSl, Wph, Wpl, Wden, Wdh, total;
};

CacheLayout make_cache_layout(const wc_problem& p, int capacity) {
  CacheLayout C{};
  const size_t H = (size_t)p.heads, lo = p.dtype == WC_F32 ? 1 : 0;
  C.cp = wc::attend_rows(capacity);
  const size_t cp = (size_t)C.cp;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  C.KSh = take(H * cp * p.d * 2);
  C.KSl = take(lo * H * cp * p.d * 2);
  C.Wph = take(H * p.dv * cp * 2);
  C.Wpl = take(lo * H * p.dv * cp * 2);
  C.Wden = take(H * cp * 4);
  C.Wdh = take(H * cp * 2);
  C.total = off;
  return C;
}

// The attention arguments that address a cache.
wc::AttendArgs cache_args(const wc_problem& p, const CacheLayout& C, const void* cache, int capacity) {
  wc::AttendArgs a{};
  char* c = static_cast<char*>(const_cast<void*>(cache));
  a.bf16 = p.dtype == WC_BF16;
  a.H = p.heads; a.d = p.d; a.dv = p.dv; a.r = capacity;
  a.beta_log2e = beta_log2e(p.d);
  a.ldrows = C.cp;
  a.KSh = reinterpret_cast<uint16_t*>(c + C.KSh);
  a.KSl = p.dtype == WC_F32 ? reinterpret_cast<uint16_t*>(c + C.KSl) : nullptr;
  a.Wph = reinterpret_cast<uint16_t*>(c + C.Wph);
  a.Wpl = p.dtype == WC_F32 ? reinterpret_cast<uint16_t*>(c + C.Wpl) : nullptr;
  a.Wden = reinterpret_cast<float*>(c + C.Wden);
  a.Wdh = reinterpret_cast<uint16_t*>(c + C.Wdh);
  return a;
}

// A few bf16 queries per head take the decode kernel; more queries, or fp32, the attention
// kernels with the coreset split.
bool decode_kernel_path(const wc_problem& p) { return p.dtype == WC_BF16 && p.m <= wc::kDecodeMaxQueries; }

size_t decode_ws_bytes(const wc_problem& p, int rows) {
  const int ns = decode_kernel_path(p) ? wc::decode_splits(rows) : attend_split(p, (size_t)p.m, (size_t)rows);
  return ns > 1 ? align_up((size_t)p.heads * ns * p.m * (p.dv + 1) * 4) : 0;
}

}  // namespace

namespace wc {

wc_status forward_check(const wc_problem* p, const void* Q, const void* K, const void* V,
                        const float* u_forced, const void* O, const int32_t* pivots,
                        const int32_t* rank, const uint32_t* flags) {
  const wc_status st = check_problem(p);
  if (st != WC_OK || p->heads == 0) return st;
  if (!req(K) || !req(V) || !req(rank) || !req(flags) || !opt(u_forced) || !opt(pivots))
    return WC_ERR_INVALID_ARG;
  if (p->m > 0 && (!req(Q) || !req(O))) return WC_ERR_INVALID_ARG;
  return WC_OK;
}

}  // namespace wc

extern "C" {

int32_t wc_abi_version(void) { return WC_ABI_VERSION; }

const char* wc_status_string(wc_status s) {
  switch (s) {
    case WC_OK: return "ok";
    case WC_ERR_INVALID_ARG: return "invalid argument";
    case WC_ERR_UNSUPPORTED: return "unsupported problem (d, dv, dtype or size)";
    case WC_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case WC_ERR_DEVICE: return "HIP launch or runtime error";
  }
  return "unknown status";
}

wc_status wc_workspace_bytes(const wc_problem* p, size_t* bytes) {
  const wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (!bytes) return WC_ERR_INVALID_ARG;
  *bytes = p->heads == 0 ? 0 : workspace_total(*p);
  return WC_OK;
}

wc_status wc_rpcholesky(const wc_problem* p, const void* K, const float* u_forced,
                        uint64_t seed, int32_t* pivots, float* F, float* diag, double* trace,
                        int32_t* rank, uint32_t* flags, void* ws, size_t ws_bytes,
                        void* stream) {
  wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (centred(*p)) return WC_ERR_UNSUPPORTED;  // wc_forward only
  if (binned(*p)) return WC_ERR_UNSUPPORTED;
  if (p->heads == 0) return WC_OK;
  if (!req(K) || !req(pivots) || !req(F) || !req(rank) || !req(flags) || !opt(u_forced) ||
      !opt(diag) || !opt(trace))
    return WC_ERR_INVALID_ARG;
  Layout L;
  if ((st = check_ws(*p, ws, ws_bytes, &L)) != WC_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (blocked(*p))
    return dev(run_rpc_block(*p, L, ws, K, u_forced, seed, pivots, F, diag, trace, rank, flags, s));
  if (resident_ok(*p)) {
    wc::ResidentArgs a{};
    a.K = static_cast<const uint16_t*>(K);
    a.u_forced = u_forced; a.seed = seed;
    a.n = p->n; a.m = p->m; a.r = p->r;
    a.beta_log2e = beta_log2e(p->d);
    a.pivots = pivots; a.F = F; a.diag = diag; a.trace = trace; a.rank = rank; a.flags = flags;
    return dev(wc::launch_resident(a, p->heads, p->d, p->dv, s));
  }
  return dev(run_rpc_stream(*p, L, ws, K, u_forced, seed, pivots, F, diag, trace, rank, flags, s));
}

wc_status wc_weights(const wc_problem* p, const void* V, const int32_t* pivots,
                     const int32_t* rank, const float* F, float* W, void* ws, size_t ws_bytes,
                     void* stream) {
  wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (centred(*p)) return WC_ERR_UNSUPPORTED;  // wc_forward only
  if (binned(*p)) return WC_ERR_UNSUPPORTED;
  if (p->heads == 0) return WC_OK;
  if (!req(V) || !req(pivots) || !req(rank) || !req(F) || !req(W)) return WC_ERR_INVALID_ARG;
  Layout L;
  if ((st = check_ws(*p, ws, ws_bytes, &L)) != WC_OK) return st;
  return dev(run_weights(*p, L, ws, V, pivots, rank, F, W, static_cast<hipStream_t>(stream)));
}

wc_status wc_weights_keys_workspace_bytes(const wc_problem* p, size_t* bytes) {
  const wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (centred(*p) || binned(*p)) return WC_ERR_UNSUPPORTED;
  if (!bytes) return WC_ERR_INVALID_ARG;
  *bytes = p->heads == 0 ? 0 : make_union_layout(*p, 0).total;
  return WC_OK;
}

wc_status wc_weights_keys(const wc_problem* p, const void* K, const void* V, const int32_t* pivots,
                          const int32_t* rank, float* W, uint32_t* flags, void* ws, size_t ws_bytes,
                          void* stream) {
  wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (centred(*p) || binned(*p)) return WC_ERR_UNSUPPORTED;
  if (p->heads == 0) return WC_OK;
  if (!req(K) || !req(V) || !req(pivots) || !req(rank) || !req(W) || !req(flags)) return WC_ERR_INVALID_ARG;
  const UnionLayout U = make_union_layout(*p, 0);
  if (!ws || !aligned16(ws) || ws_bytes < U.total) return WC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* piv = at<int32_t>(ws, U.piv);
  hipError_t e = wc::launch_union_mask(pivots, rank, piv, p->heads, p->r, s);
  if (e == hipSuccess) e = run_union_weights(*p, U, ws, K, V, piv, W, flags, s);
  return dev(e);
}

wc_status wc_attend(const wc_problem* p, const void* Q, const void* K, const int32_t* pivots,
                    const int32_t* rank, const float* W, void* O, uint32_t* flags, void* ws,
                    size_t ws_bytes, void* stream) {
  wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (centred(*p)) return WC_ERR_UNSUPPORTED;  // wc_forward only
  if (binned(*p)) return WC_ERR_UNSUPPORTED;
  if (p->heads == 0) return WC_OK;
  if (!req(K) || !req(pivots) || !req(rank) || !req(W) || !req(flags)) return WC_ERR_INVALID_ARG;
  if (p->m > 0 && (!req(Q) || !req(O))) return WC_ERR_INVALID_ARG;
  Layout L;
  if ((st = check_ws(*p, ws, ws_bytes, &L)) != WC_OK) return st;
  return dev(run_attend(*p, L, ws, Q, K, pivots, rank, W, O, flags, static_cast<hipStream_t>(stream)));
}

wc_status wc_forward(const wc_problem* p, const void* Q, const void* K, const void* V,
                     const float* u_forced, uint64_t seed, void* O, int32_t* pivots,
                     int32_t* rank, uint32_t* flags, void* ws, size_t ws_bytes, void* stream) {
  wc_status st = wc::forward_check(p, Q, K, V, u_forced, O, pivots, rank, flags);
  if (st != WC_OK || p->heads == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (centred(*p)) {
    // every step below runs on the centred keys, kept after the forward's own workspace
    if (!ws || !aligned16(ws) || ws_bytes < workspace_total(*p)) return WC_ERR_WORKSPACE;
    const size_t base = binned(*p) ? make_binned_layout(*p).total : make_layout(*p).total;
    const CenterLayout C = make_center_layout(*p, base);
    wc::CenterArgs c{};
    c.K = K; c.bf16 = p->dtype == WC_BF16;
    c.H = p->heads; c.n = p->n; c.d = p->d; c.nblk = wc::center_blocks(p->n);
    c.part = at<double>(ws, C.part); c.mean = at<double>(ws, C.mean); c.Kc = at<void>(ws, C.Kc);
    const hipError_t e = wc::launch_center(c, s);
    if (e != hipSuccess) return dev(e);
    K = c.Kc;
  }
  if (union_path(*p)) return forward_binned(*p, Q, K, V, u_forced, seed, O, pivots, rank, flags, ws, ws_bytes, s);
  Layout L;
  if ((st = check_ws(*p, ws, ws_bytes, &L)) != WC_OK) return st;
  if (resident_ok(*p) && p->m > 0) {
    wc::ResidentArgs a{};
    a.Q = static_cast<const uint16_t*>(Q);
    a.K = static_cast<const uint16_t*>(K);
    a.V = static_cast<const uint16_t*>(V);
    a.u_forced = u_forced; a.seed = seed;
    a.n = p->n; a.m = p->m; a.r = p->r;
    a.beta_log2e = beta_log2e(p->d);
    a.O = static_cast<uint16_t*>(O);
    a.pivots = pivots; a.rank = rank; a.flags = flags;
    return dev(wc::launch_resident(a, p->heads, p->d, p->dv, s));
  }
  int32_t* piv = pivots ? pivots : at<int32_t>(ws, L.piv);
  float* F = at<float>(ws, L.F);
  float* W = at<float>(ws, L.W);
  hipError_t e = run_select(*p, L, ws, K, u_forced, seed, piv, F, rank, flags, s);
  if (e == hipSuccess) e = run_weights(*p, L, ws, V, piv, rank, F, W, s, flags);
  if (e == hipSuccess) e = run_attend(*p, L, ws, Q, K, piv, rank, W, O, flags, s);
  return dev(e);
}

wc_status wc_cache_bytes(const wc_problem* p, int32_t capacity, size_t* bytes) {
  const wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (!bytes || capacity < 1) return WC_ERR_INVALID_ARG;
  *bytes = p->heads == 0 ? 0 : make_cache_layout(*p, capacity).total;
  return WC_OK;
}

wc_status wc_compress(const wc_problem* p, const void* K, const void* V, const float* u_forced,
                      uint64_t seed, void* cache, int32_t capacity, int32_t* pivots, int32_t* rank,
                      uint32_t* flags, void* ws, size_t ws_bytes, void* stream) {
  wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (centred(*p)) return WC_ERR_UNSUPPORTED;  // wc_forward only
  if (capacity < p->r) return WC_ERR_INVALID_ARG;
  if (p->heads == 0) return WC_OK;
  if (!req(K) || !req(V) || !req(cache) || !req(rank) || !req(flags) || !opt(u_forced) || !opt(pivots))
    return WC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  wc_problem q = *p;
  q.m = 0;
  const CacheLayout C = make_cache_layout(q, capacity);
  wc::AttendArgs a = cache_args(q, C, cache, capacity);
  a.K = K; a.n = q.n; a.r = q.r;
  hipError_t e;
  if (union_path(q)) {
    // selection and weights as in the forward (no queries); the weights and the head's
    // pivots are left in the workspace
    if ((st = forward_binned(q, nullptr, K, V, u_forced, seed, nullptr, pivots, rank, flags, ws, ws_bytes, s)) != WC_OK)
      return st;
    const BinnedLayout B = make_binned_layout(q);
    a.pivots = pivots ? pivots : at<int32_t>(ws, B.piv);
    a.rank = at<int32_t>(ws, B.rank_slots);
    a.W = at<float>(ws, B.sub.W);
  } else {
    Layout L;
    if ((st = check_ws(q, ws, ws_bytes, &L)) != WC_OK) return st;
    int32_t* piv = pivots ? pivots : at<int32_t>(ws, L.piv);
    float* F = at<float>(ws, L.F);
    float* W = at<float>(ws, L.W);
    e = run_select(q, L, ws, K, u_forced, seed, piv, F, rank, flags, s);
    if (e == hipSuccess) e = run_weights(q, L, ws, V, piv, rank, F, W, s, flags);
    if (e != hipSuccess) return dev(e);
    a.pivots = piv; a.rank = rank; a.W = W;
  }
  // every staged row is written: the coreset rows, then zeros up to the capacity
  a.ldrows = C.cp;
  return dev(wc::launch_attend_prep(a, s));
}

wc_status wc_cache_append(const wc_problem* p, const void* K_new, const void* V_new, int32_t count,
                          int32_t row0, void* cache, int32_t capacity, void* stream) {
  const wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (centred(*p)) return WC_ERR_UNSUPPORTED;  // wc_forward only
  if (count < 0 || row0 < 0 || capacity < 1 || (int64_t)row0 + count > capacity) return WC_ERR_INVALID_ARG;
  if (p->heads == 0 || count == 0) return WC_OK;
  if (!req(K_new) || !req(V_new) || !req(cache)) return WC_ERR_INVALID_ARG;
  const CacheLayout C = make_cache_layout(*p, capacity);
  wc::AttendArgs a = cache_args(*p, C, cache, capacity);
  a.K = K_new; a.V = V_new; a.n = count; a.row0 = row0;
  return dev(wc::launch_attend_append(a, static_cast<hipStream_t>(stream)));
}

wc_status wc_decode_workspace_bytes(const wc_problem* p, int32_t rows, size_t* bytes) {
  const wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (!bytes || rows < 1) return WC_ERR_INVALID_ARG;
  *bytes = p->heads == 0 ? 0 : decode_ws_bytes(*p, rows);
  return WC_OK;
}

wc_status wc_decode(const wc_problem* p, const void* Q, const void* cache, int32_t capacity,
                    int32_t rows, void* O, uint32_t* flags, void* ws, size_t ws_bytes, void* stream) {
  const wc_status st = check_problem(p);
  if (st != WC_OK) return st;
  if (centred(*p)) return WC_ERR_UNSUPPORTED;  // wc_forward only
  if (rows < 1 || capacity < rows) return WC_ERR_INVALID_ARG;
  if (p->heads == 0 || p->m == 0) return WC_OK;
  if (!req(Q) || !req(cache) || !req(O) || !req(flags)) return WC_ERR_INVALID_ARG;
  const size_t need = decode_ws_bytes(*p, rows);
  if (need > 0 && (!ws || !aligned16(ws) || ws_bytes < need)) return WC_ERR_WORKSPACE;
  const CacheLayout C = make_cache_layout(*p, capacity);
  wc::AttendArgs a = cache_args(*p, C, cache, capacity);
  a.Q = Q; a.m = p->m; a.scan_rows = rows;
  a.O = O; a.flags = flags;
  if (decode_kernel_path(*p)) {
    a.Ypart = need > 0 ? static_cast<float*>(ws) : nullptr;
    return dev(wc::launch_decode(a, static_cast<hipStream_t>(stream)));
  }
  a.nsplit = attend_split(*p, (size_t)p->m, (size_t)rows);
  a.Ypart = a.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  return dev(wc::launch_attend_core(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
