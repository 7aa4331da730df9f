// Streaming randomly pivoted Cholesky for heads of any length (page
// gist.science/de/paper/2602.10056, "Methodik" part 1: partial Cholesky of H = exp(beta K K^T),
// each pivot drawn from the diagonal of the residual kernel matrix).
//
// One launch per pivot step covers every head; a head's n rows are split into blocks of
// `rows` rows, one workgroup each.  The kernel boundary is the only global barrier:
//   * at the start of step t every workgroup of a head reads the fp64 masses of all blocks
//     (written at step t-1), finds T and the block holding u_t T, rescans that block's
//     residual diagonal and so resolves the same pivot s as every other workgroup;
//   * it gathers k_s and F[s, :t], forms g_s = H_ss - |F[s, :t]|^2, then for its own rows
//     g_i = exp(beta k_i.k_s) - F[i, :t].F[s, :t], F[i, t] = g_i / sqrt(g_s),
//     diag_i -= F[i, t]^2 (diag_s = 0), and writes its block's new fp64 mass.
// The residual diagonal and the block masses are double-buffered so that step t reads only
// what step t-1 wrote.  Column t of F is a contiguous run of n floats (F is [r][n]), so the
// correction F[i, :t].F[s, :t] streams F column by column with coalesced loads.
#include "wc_device.h"
#include "wc_elim.h"
#include "wc_kernels.h"

namespace wc {

constexpr int NT = kStreamThreads;  // 256
constexpr int NW = NT / 64;

// ---- key dots k_i . k_s with one 16-byte piece of a key row per lane ------------------------
// A key row is KL = D sizeof(T) / 16 pieces; KL consecutive lanes read one row (a wave reads
// 64 / KL whole rows with one coalesced load), each lane forms the dot of its piece with the
// same piece of k_s, and the KL partial sums are added by an xor butterfly.  Every lane of the
// group ends with the same value, and any row, wherever it sits in a wave, is summed in the
// same order, so the pivot's own entry H_ss equals the one its column holds.
template <typename T, int D>
struct KeyPieces {
  static constexpr int KL = D * (int)sizeof(T) / 16;  // lanes per key row
  static constexpr int RPL = 64 / KL;                 // key rows per wave load
};

typedef __attribute__((ext_vector_type(4))) float v4f;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of G lanes (G = 8, 16 or 32), the result in every lane of the group.
template <int G>
__device__ __forceinline__ float group_sum(float a) {
  a += dpp_f<0xB1>(a);   // quad_perm [1, 0, 3, 2]: lane ^ 1
  a += dpp_f<0x4E>(a);   // quad_perm [2, 3, 0, 1]: lane ^ 2
  a += dpp_f<0x141>(a);  // row_half_mirror: the other quad of the 8 lanes
  if constexpr (G >= 16) a += dpp_f<0x140>(a);  // row_mirror: the other 8 lanes of the 16
  if constexpr (G >= 32) a += __shfl_xor(a, 16, 64);
  return a;
}

// Dot of one 16-byte piece of a key row with the same piece of k_s (fixed order).
__device__ __forceinline__ float piece_dot(uint4 v, uint4 k, uint16_t) {
  float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), __builtin_bit_cast(bf16x2, k.x), 0.f, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), __builtin_bit_cast(bf16x2, k.y), a, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), __builtin_bit_cast(bf16x2, k.z), a, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), __builtin_bit_cast(bf16x2, k.w), a, false);
}
__device__ __forceinline__ float piece_dot(uint4 v, uint4 k, float) {
  float a = __uint_as_float(v.x) * __uint_as_float(k.x);
  a = fmaf(__uint_as_float(v.y), __uint_as_float(k.y), a);
  a = fmaf(__uint_as_float(v.z), __uint_as_float(k.z), a);
  return fmaf(__uint_as_float(v.w), __uint_as_float(k.w), a);
}

// k_i . k_s for the key rows [r0, r0 + NT RPT) of a workgroup into s_dot (rows past n: 0).
// kpiece: this lane's piece of k_s (piece lane % KL).  Wave w takes rows r0 + 64 RPT w + ...
template <typename T, int D, int RPT>
__device__ __forceinline__ void block_key_dots(const T* K, int r0, int n, uint4 kpiece, float* s_dot) {
  using P = KeyPieces<T, D>;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int c = lane % P::KL, sub = lane / P::KL;
  const int w0 = wid * 64 * RPT;
  const uint4* Kp = reinterpret_cast<const uint4*>(K);
#pragma unroll 8
  for (int k = 0; k < RPT * P::KL; ++k) {
    const int row = r0 + w0 + k * P::RPL + sub;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < n) v = Kp[(size_t)row * P::KL + c];
    const float a = group_sum<P::KL>(piece_dot(v, kpiece, T{}));
    if (c == 0) s_dot[w0 + k * P::RPL + sub] = a;
  }
}

// Each step reads F[:, :t] once.  When the whole factor is larger than the 256 MB last-level
// cache (MALL) it comes from HBM every step anyway, and nontemporal loads keep the stream from
// displacing the keys and the residual; a smaller factor stays cached between steps and is
// read with ordinary loads.
constexpr size_t kMallBytes = size_t(256) << 20;
// RPT contiguous floats (RPT = 4: one 16-byte access; the caller guarantees alignment).
template <int RPT>
__device__ __forceinline__ void load_rows(const float* p, float* v) {
  if constexpr (RPT == 4) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int e = 0; e < RPT; ++e) v[e] = p[e];
  }
}
template <int RPT, bool NTL>
__device__ __forceinline__ void load_factor_rows(const float* p, float* v) {
  if constexpr (!NTL) {
    load_rows<RPT>(p, v);
  } else if constexpr (RPT == 4) {
    const v4f x = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int e = 0; e < RPT; ++e) v[e] = __builtin_nontemporal_load(p + e);
  }
}
template <int RPT>
__device__ __forceinline__ void store_rows(float* p, const float* v) {
  if constexpr (RPT == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int e = 0; e < RPT; ++e) p[e] = v[e];
  }
}

// Block-wide fp64 sum in a fixed order (wave trees, then waves in order); all threads get it.
__device__ __forceinline__ double block_sum(double x, double* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  x = wave_sum(x);
  __syncthreads();
  if (lane == 0) red[wid] = x;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red[w];
  return s;
}

// Block-wide exclusive scan of one fp64 value per thread (thread order); returns the
// exclusive prefix, and the total through *tot.  Fixed order, identical in every workgroup.
__device__ __forceinline__ double block_excl_scan(double x, double* red, double* tot) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const double inc = wave_incl_scan(x);
  __syncthreads();
  if (lane == 63) red[wid] = inc;
  __syncthreads();
  double pre = 0.0, all = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w == wid) pre = all;
    all += red[w];
  }
  *tot = all;
  return pre + (inc - x);
}

__device__ __forceinline__ int block_min_int(int v, int* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, 64));
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  int s = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) s = min(s, red[w]);
  return s;
}
__device__ __forceinline__ int block_max_int(int v, int* red) {
  return -block_min_int(-v, red);
}

// Pivot uniforms of every (head, step), drawn once before the loop.
__global__ void __launch_bounds__(256) uniforms_kernel(StreamRpcArgs a) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)a.H * a.r) return;
  a.uniforms[e] = philox_uniform(a.seed, (uint32_t)(e / a.r), (uint32_t)(e % a.r));
}

// Initial residual diag_i = exp(beta |k_i|^2) and per-block masses.  Eight lanes share a key
// row (16-byte loads, so a wave reads eight whole rows contiguously), then combine their
// partial squared norms.
template <typename T, int D>
__global__ void __launch_bounds__(NT) rpc_init_kernel(StreamRpcArgs a, int rows) {
  __shared__ double red[NW];
  constexpr int PER = D / 8;                        // elements per lane
  constexpr int E = 16 / (int)sizeof(T);            // elements per 16-byte load
  const int h = blockIdx.y, b = blockIdx.x, tid = threadIdx.x, sub = tid & 7, grp = tid >> 3;
  const T* K = reinterpret_cast<const T*>(a.K) + (size_t)h * a.n * D;
  double mass = 0.0;
  for (int k = 0; k < rows; k += NT / 8) {
    const int i = b * rows + k + grp;
    float ss = 0.f;
    if (i < a.n) {
      const T* kr = K + (size_t)i * D + sub * PER;
#pragma unroll
      for (int q = 0; q < PER / E; ++q) {
        T x[E];
        *reinterpret_cast<uint4*>(x) = *reinterpret_cast<const uint4*>(kr + q * E);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float v = ld_elem<T>(x + e);
          ss = fmaf(v, v, ss);
        }
      }
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    if (sub == 0 && i < a.n) {
      const float d0 = __builtin_amdgcn_exp2f(ss * a.beta_log2e);
      a.diag0[(size_t)h * a.n + i] = d0;
      mass += mass_of(d0);
    }
  }
  const double tot = block_sum(mass, red);
  if (tid == 0) {
    a.part0[(size_t)h * a.nblk + b] = tot;
    if (b == 0) {
      a.rank[h] = a.r;
      a.flags[h] = 0u;
    }
  }
}

template <typename T, int D, int RPT, bool NTL>
__global__ void __launch_bounds__(NT) rpc_step_kernel(StreamRpcArgs a, int rows, int t) {
  __shared__ double red[NW];
  __shared__ int ired[NW];
  __shared__ __attribute__((aligned(16))) float s_dot[NT * RPT];
  extern __shared__ __attribute__((aligned(16))) double s_dyn[];
  double* s_part = s_dyn;                                   // [nblk]
  float* s_fs = reinterpret_cast<float*>(s_dyn + a.nblk);   // [r]
  const int h = blockIdx.y, b = blockIdx.x, tid = threadIdx.x;
  // the loads that depend on nothing go out together, before the first test: the head's rank,
  // this step's uniform and (below) the block masses
  const int rk = a.rank[h];
  const float u_t = a.uniforms[(size_t)h * a.r + t];
  const int n = a.n, nblk = a.nblk;
  const double* part = (t & 1) ? a.part1 : a.part0;
  double* part_nx = (t & 1) ? a.part0 : a.part1;
  const float* dg_in = ((t & 1) ? a.diag1 : a.diag0) + (size_t)h * n;
  float* dg_out = ((t & 1) ? a.diag0 : a.diag1) + (size_t)h * n;
  const T* K = reinterpret_cast<const T*>(a.K) + (size_t)h * n * D;
  float* F = a.F + (size_t)h * a.r * n;

  // ---- 1. total mass T and the block holding u_t T ----
  // thread tid owns the contiguous run of blocks [tid*per, tid*per + per)
  const int per = (nblk + NT - 1) / NT;
  double mine = 0.0;
  for (int e = 0; e < per; ++e) {
    const int bb = tid * per + e;
    if (bb < nblk) {
      const double v = part[(size_t)h * nblk + bb];
      s_part[bb] = v;
      mine += v;
    }
  }
  if (rk < t) return;  // this head broke down at an earlier step
  double Ttot;
  const double excl = block_excl_scan(mine, red, &Ttot);
  const bool lead = (b == 0 && tid == 0);
  if (!(Ttot > 0.0) || !__builtin_isfinite(Ttot)) {
    if (lead) {
      a.rank[h] = t;
      a.flags[h] |= WC_DFLAG_BREAKDOWN | (__builtin_isfinite(Ttot) ? 0u : WC_DFLAG_NONFINITE);
      if (a.trace) a.trace[(size_t)h * (a.r + 1) + t] = __builtin_isfinite(Ttot) ? Ttot : 0.0;
    }
    return;
  }
  const double uT = (double)u_t * Ttot;
  int cand = 0x7fffffff, lastpos = -1;
  double run = excl;
  for (int e = 0; e < per; ++e) {
    const int bb = tid * per + e;
    if (bb < nblk) {
      const double v = s_part[bb];
      run += v;
      if (cand == 0x7fffffff && v > 0.0 && run > uT) cand = bb;
      if (v > 0.0) lastpos = bb;
    }
  }
  int bstar = block_min_int(cand, ired);
  if (bstar == 0x7fffffff) bstar = block_max_int(lastpos, ired);
  // exclusive offset of block bstar, recomputed in the same order as `run`
  __syncthreads();
  if (tid == bstar / per) {
    double o = excl;
    for (int e = 0; e < bstar - tid * per; ++e) o += s_part[tid * per + e];
    red[0] = o;
  }
  __syncthreads();
  const double boff = red[0];

  // ---- 2. the pivot row inside block bstar ----
  // thread tid owns rows [r0 + tid*rpt, r0 + tid*rpt + rpt)
  const int rpt = rows / NT;
  const int r0 = bstar * rows;
  double pm[4];
  double tmass = 0.0;
  for (int e = 0; e < rpt; ++e) {
    const int i = r0 + tid * rpt + e;
    pm[e] = (i < n) ? mass_of(dg_in[i]) : 0.0;
    tmass += pm[e];
  }
  double btot;
  __syncthreads();
  const double rexcl = block_excl_scan(tmass, red, &btot);
  int scand = 0x7fffffff, slast = -1;
  double c = boff + rexcl;
  for (int e = 0; e < rpt; ++e) {
    c += pm[e];
    const int i = r0 + tid * rpt + e;
    if (scand == 0x7fffffff && c > uT && pm[e] > 0.0) scand = i;
    if (pm[e] > 0.0) slast = i;
  }
  int s = block_min_int(scand, ired);
  if (s == 0x7fffffff) s = block_max_int(slast, ired);
  if (s < 0 || s >= n) {  // no row with mass in the selected block: cannot happen for finite T > 0
    if (lead) {
      a.rank[h] = t;
      a.flags[h] |= WC_DFLAG_BREAKDOWN | WC_DFLAG_NONFINITE;
    }
    return;
  }

  // ---- 3. gather k_s (this lane's piece) and F[s, :t]; g_s ----
  const uint4 kpiece = reinterpret_cast<const uint4*>(K + (size_t)s * D)[(threadIdx.x & 63) % KeyPieces<T, D>::KL];
  double sq = 0.0;
  for (int j = tid; j < t; j += NT) {
    const float v = F[(size_t)j * n + s];
    s_fs[j] = v;
  }
  __syncthreads();
  float hss = 0.f;
  {
    float part_sq = 0.f;
    for (int j = tid; j < t; j += NT) part_sq = fmaf(s_fs[j], s_fs[j], part_sq);
    sq = (double)part_sq;
  }
  const double sqt = block_sum(sq, red);
  hss = __builtin_amdgcn_exp2f(group_sum<KeyPieces<T, D>::KL>(piece_dot(kpiece, kpiece, T{})) * a.beta_log2e);
  const float gs = hss - (float)sqt;
  if (!(gs > 0.f) || !__builtin_isfinite(gs)) {
    if (lead) {
      a.rank[h] = t;
      a.flags[h] |= WC_DFLAG_BREAKDOWN | (__builtin_isfinite(gs) ? 0u : WC_DFLAG_NONFINITE);
      if (a.trace) a.trace[(size_t)h * (a.r + 1) + t] = Ttot;
    }
    return;
  }
  if (lead) {
    a.pivots[(size_t)h * a.r + t] = s;
    if (a.trace) a.trace[(size_t)h * (a.r + 1) + t] = Ttot;
  }
  const float rs = 1.0f / sqrtf(gs);

  // ---- 4. this block's rows: new column of F, residual update, block mass ----
  // Thread tid owns the RPT contiguous rows i0 .. i0 + RPT - 1, so column j of F arrives as one
  // RPT-wide load per thread and a wave reads RPT * 256 contiguous bytes; U columns are in
  // flight at once to keep enough bytes outstanding per CU for HBM.
  double mass = 0.0;
  const int i0 = b * rows + tid * RPT;
  block_key_dots<T, D, RPT>(K, b * rows, n, kpiece, s_dot);
  __syncthreads();
  if (i0 < n) {
    float hcol[RPT];
#pragma unroll
    for (int e = 0; e < RPT; ++e) hcol[e] = __builtin_amdgcn_exp2f(s_dot[tid * RPT + e] * a.beta_log2e);
    float acc[RPT];
#pragma unroll
    for (int e = 0; e < RPT; ++e) acc[e] = 0.f;
    constexpr int U = RPT == 4 ? 8 : 16;
    const float* Fi = F + i0;
    int j = 0;
    for (; j + U <= t; j += U) {
      float fv[U][RPT];
#pragma unroll
      for (int u = 0; u < U; ++u) load_factor_rows<RPT, NTL>(Fi + (size_t)(j + u) * n, fv[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float fs = s_fs[j + u];
#pragma unroll
        for (int e = 0; e < RPT; ++e) acc[e] = fmaf(fv[u][e], fs, acc[e]);
      }
    }
    for (; j < t; ++j) {
      float fv[RPT];
      load_factor_rows<RPT, NTL>(Fi + (size_t)j * n, fv);
      const float fs = s_fs[j];
#pragma unroll
      for (int e = 0; e < RPT; ++e) acc[e] = fmaf(fv[e], fs, acc[e]);
    }
    float f[RPT], din[RPT], dnew[RPT];
    load_rows<RPT>(dg_in + i0, din);
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      f[e] = (hcol[e] - acc[e]) * rs;
      dnew[e] = (i0 + e == s) ? 0.f : din[e] - f[e] * f[e];
      mass += mass_of(dnew[e]);
    }
    store_rows<RPT>(F + (size_t)t * n + i0, f);
    store_rows<RPT>(dg_out + i0, dnew);
  }
  const double tot = block_sum(mass, red);
  if (tid == 0) part_nx[(size_t)h * nblk + b] = tot;
}

// Final bookkeeping per head: trace after the last step, -1 pivots and zero F columns
// after a breakdown, copy of the final residual diagonal.
template <int DUMMY>
__global__ void __launch_bounds__(NT) rpc_final_kernel(StreamRpcArgs a) {
  __shared__ double red[NW];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int rk = a.rank[h];
  const int n = a.n, nblk = a.nblk;
  const double* part = (rk & 1) ? a.part1 : a.part0;
  const float* dg = ((rk & 1) ? a.diag1 : a.diag0) + (size_t)h * n;
  if (rk == a.r && a.trace) {
    const int per = (nblk + NT - 1) / NT;
    double mine = 0.0;
    for (int e = 0; e < per; ++e) {
      const int bb = tid * per + e;
      if (bb < nblk) mine += part[(size_t)h * nblk + bb];
    }
    double T;
    block_excl_scan(mine, red, &T);
    if (tid == 0) a.trace[(size_t)h * (a.r + 1) + a.r] = T;
  }
  if (a.trace)
    for (int t = rk + 1 + tid; t <= a.r; t += NT) a.trace[(size_t)h * (a.r + 1) + t] = 0.0;
  for (int t = rk + tid; t < a.r; t += NT) a.pivots[(size_t)h * a.r + t] = -1;
  for (size_t e = (size_t)rk * n + tid; e < (size_t)a.r * n; e += NT) a.F[(size_t)h * a.r * n + e] = 0.f;
  if (a.diag_out)
    for (int i = tid; i < n; i += NT) a.diag_out[(size_t)h * n + i] = dg[i];
}

template <typename T, int D>
static hipError_t run_rpc(StreamRpcArgs a, int rows, hipStream_t st) {
  const dim3 grid(a.nblk, a.H);
  const size_t lds = (size_t)a.nblk * sizeof(double) + (size_t)a.r * sizeof(float);
  hipError_t e;
  if (!a.u_forced) {
    const size_t nu = (size_t)a.H * a.r;
    hipLaunchKernelGGL(uniforms_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((rpc_init_kernel<T, D>), grid, dim3(NT), 0, st, a, rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool nt = (size_t)a.H * a.r * a.n * sizeof(float) > kMallBytes;
  for (int t = 0; t < a.r; ++t) {
    if (rows == 4 * NT && nt)
      hipLaunchKernelGGL((rpc_step_kernel<T, D, 4, true>), grid, dim3(NT), lds, st, a, rows, t);
    else if (rows == 4 * NT)
      hipLaunchKernelGGL((rpc_step_kernel<T, D, 4, false>), grid, dim3(NT), lds, st, a, rows, t);
    else if (nt)
      hipLaunchKernelGGL((rpc_step_kernel<T, D, 1, true>), grid, dim3(NT), lds, st, a, rows, t);
    else
      hipLaunchKernelGGL((rpc_step_kernel<T, D, 1, false>), grid, dim3(NT), lds, st, a, rows, t);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((rpc_final_kernel<0>), dim3(a.H), dim3(NT), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Block pivot selection (b candidates per round; the pages leave the mechanism that would lift
// the sequential pivot selection to future work, gist.science/de/paper/2602.10056, "Bedeutung
// und Ansprueche"; read here as the block variant of randomly pivoted Cholesky, oversampled
// until the r slots are full).  Round k reads the residual and block masses its predecessor
// wrote; f0 slots are full when it starts:
//   sample  one workgroup per candidate resolves s_j = min{i : C_i > u T} on that residual,
//           u = uniforms[k b + j];
//   column  G[:, j] = exp(beta K k_{s_j}) - F[:, :f0] F[s_j, :f0]^T for all rows (F is read
//           once per round instead of once per pivot);
//   factor  the b x b block G[S, :] is eliminated in candidate order with the leave-out rule
//           (elim_block, relative to H_ss); the kept candidates take slots f0, f0 + 1, ...
//           while slots remain;
//   apply   F[:, slot_j] = (G M^T)[:, j] for the candidates with a slot, residual, masses.
// Rounds run until the slots are full or kBlockDraws r candidates are drawn; every kernel of
// a head that is full, or has stopped, returns at once.
// ---------------------------------------------------------------------------------------------

__global__ void __launch_bounds__(256) blk_uniforms_kernel(BlockRpcArgs A) {
  const StreamRpcArgs& a = A.s;
  const size_t per = (size_t)kBlockDraws * a.r;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)a.H * per) return;
  a.uniforms[e] = philox_uniform(a.seed, (uint32_t)(e / per), (uint32_t)(e % per));
}

__global__ void __launch_bounds__(NT) blk_init_kernel(BlockRpcArgs A) {
  const StreamRpcArgs& a = A.s;
  const int h = blockIdx.x;
  if (threadIdx.x == 0) {
    a.rank[h] = 0;
    A.rounds[h] = 0;
  }
  if (a.trace)
    for (int t = threadIdx.x; t <= a.r; t += NT) a.trace[(size_t)h * (a.r + 1) + t] = 0.0;
}

__device__ __forceinline__ bool blk_done(const BlockRpcArgs& A, int h) {
  return A.s.rank[h] >= A.s.r || (A.s.flags[h] & WC_DFLAG_BREAKDOWN);
}

__device__ __forceinline__ double lane_d(double x, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
  return __hiloint2double(hi, lo);
}
// The value of the lowest (or highest) lane for which `has` holds, or `none`: the minimum (or
// maximum) over the wave of a quantity that increases with the lane, by one ballot instead of a
// shuffle tree.
__device__ __forceinline__ int first_lane_value(bool has, int v, int none) {
  const uint64_t m = __ballot(has);
  return m ? __builtin_amdgcn_readlane(v, __builtin_ctzll(m)) : none;
}
__device__ __forceinline__ int last_lane_value(bool has, int v, int none) {
  const uint64_t m = __ballot(has);
  return m ? __builtin_amdgcn_readlane(v, 63 - __builtin_clzll(m)) : none;
}

// One wave per head draws the round's b candidates one after the other, without replacement:
// candidate j is the inverse-CDF draw on the round-start masses with the earlier candidates'
// masses removed.  The running sums are not rebuilt: the target u T' (T' the mass left) is
// moved past the intervals [C_{d-1}, C_d) of the earlier candidates d, taken in index order,
// and then searched on the unchanged block masses and rows.  The block masses and their
// exclusive sums sit in LDS for the round and the drawn candidates in registers (lane q the
// q-th in index order); a draw is a wave scan for the shifted target, a wave search over the
// blocks, one load of the chosen block's rows (RPT per lane), a wave scan and a shuffle to
// insert the new candidate, with no barrier.  NBR > 0: the sub-head has at most NBR blocks,
// whose rows the wave loads into registers once, before the draws (all requested together), so
// that a draw picks the chosen block's rows from registers instead of waiting on a load.
template <int RPT, int NBR>
__global__ void __launch_bounds__(64) blk_sample_kernel(BlockRpcArgs A, int k) {
  extern __shared__ __attribute__((aligned(16))) double s_blk[];  // [nblk] masses, [nblk] exclusive sums
  const StreamRpcArgs& a = A.s;
  const int h = blockIdx.x, lane = threadIdx.x;
  const int n = a.n, nblk = a.nblk, B = A.b;
  int32_t* cand = A.cand + (size_t)h * B;
  if (blk_done(A, h)) return;
  double* s_part = s_blk;
  double* s_pre = s_blk + nblk;
  const double* part = ((k & 1) ? a.part1 : a.part0) + (size_t)h * nblk;
  const float* dg_in = ((k & 1) ? a.diag1 : a.diag0) + (size_t)h * n;
  const int per = (nblk + 63) / 64;
  float dres[NBR > 0 ? NBR : 1][RPT];
  if constexpr (NBR > 0) {
#pragma unroll
    for (int q = 0; q < NBR; ++q)
#pragma unroll
      for (int e = 0; e < RPT; ++e) dres[q][e] = dg_in[min(q * 64 * RPT + lane * RPT + e, n - 1)];
  }
  double mine = 0.0;
  for (int e = 0; e < per; ++e) {
    const int bb = lane * per + e;
    if (bb < nblk) {
      const double v = part[bb];
      s_part[bb] = v;
      mine += v;
    }
  }
  const double incl = wave_incl_scan(mine);
  const double Ttot = lane_d(incl, 63);
  {
    double run = incl - mine;
    for (int e = 0; e < per; ++e) {
      const int bb = lane * per + e;
      if (bb < nblk) {
        s_pre[bb] = run;
        run += s_part[bb];
      }
    }
  }
  const int f0 = a.rank[h];
  if (!(Ttot > 0.0) || !__builtin_isfinite(Ttot)) {
    // no mass left: the loop stops (every later kernel of the head sees the flag or cand -1)
    if (lane == 0) {
      a.flags[h] |= WC_DFLAG_BREAKDOWN | (__builtin_isfinite(Ttot) ? 0u : WC_DFLAG_NONFINITE);
      if (a.trace) a.trace[(size_t)h * (a.r + 1) + f0] = __builtin_isfinite(Ttot) ? Ttot : 0.0;
    }
    for (int j = lane; j < B; j += 64) cand[j] = -1;
    return;
  }
  if (lane == 0 && a.trace) a.trace[(size_t)h * (a.r + 1) + f0] = Ttot;
  const float* u = a.uniforms + (size_t)h * kBlockDraws * a.r + (size_t)k * B;
  double removed = 0.0;
  int nd = 0;
  // the drawn candidates in index order, lane q holding the q-th: index, running sum before
  // it and its mass
  int c_idx = 0x7fffffff;
  double c_lo = 0.0, c_m = 0.0;
  for (int j = 0; j < B; ++j) {
    const double Tl = Ttot - removed;
    if (!(Tl > 0.0)) {  // every index with mass is drawn: the round has fewer candidates
      for (int jj = j + lane; jj < B; jj += 64) cand[jj] = -1;
      break;
    }
    // Move the target past the earlier candidates' intervals in index order: with M_q the
    // masses of the first q of them, the target ends at x + M_Q for the first Q whose interval
    // x + M_Q does not reach (intervals in index order start in increasing order).
    const double x0 = (double)u[j] * Tl;
    const double mq = lane < nd ? c_m : 0.0;
    const double Mx = wave_incl_scan(mq) - mq;  // M_lane
    const uint64_t stop = __ballot(lane < nd && !(x0 + Mx >= c_lo)) | (nd < 64 ? (1ull << nd) : 0ull);
    const int Q = stop ? __builtin_ctzll(stop) : 64;
    const double x = Q == 0 ? x0 : x0 + lane_d(Mx + mq, Q - 1);
    // block holding x (the last block with mass if rounding put x at or past the total)
    int bc = 0x7fffffff, lastpos = -1;
    for (int e = 0; e < per; ++e) {
      const int bb = lane * per + e;
      if (bb < nblk) {
        const double v = s_part[bb];
        if (bc == 0x7fffffff && v > 0.0 && s_pre[bb] + v > x) bc = bb;
        if (v > 0.0) lastpos = bb;
      }
    }
    // blocks go to the lanes in index order: the wave's first such block is the lowest lane's
    int bstar = first_lane_value(bc != 0x7fffffff, bc, 0x7fffffff);
    if (bstar == 0x7fffffff) bstar = last_lane_value(lastpos >= 0, lastpos, -1);
    if (bstar < 0) {  // no block with mass (excluded by T > 0; kept as a guard)
      for (int jj = j + lane; jj < B; jj += 64) cand[jj] = -1;
      break;
    }
    // row inside it: unconditional loads (clamped indices), rows past n weigh nothing
    const int r0 = bstar * 64 * RPT;
    float dv[RPT];
    if constexpr (NBR > 0) {
#pragma unroll
      for (int e = 0; e < RPT; ++e) {
        float v = dres[0][e];
#pragma unroll
        for (int q = 1; q < NBR; ++q) v = bstar == q ? dres[q][e] : v;
        dv[e] = v;
      }
    } else {
#pragma unroll
      for (int e = 0; e < RPT; ++e) dv[e] = dg_in[min(r0 + lane * RPT + e, n - 1)];
    }
    double pm[RPT];
    double tmass = 0.0;
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      pm[e] = (r0 + lane * RPT + e < n) ? mass_of(dv[e]) : 0.0;
      tmass += pm[e];
    }
    const double rincl = wave_incl_scan(tmass);
    const double base = s_pre[bstar] + (rincl - tmass);
    int scand = 0x7fffffff;
    double c = base;
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      c += pm[e];
      if (scand == 0x7fffffff && c > x && pm[e] > 0.0) scand = r0 + lane * RPT + e;
    }
    const int s = first_lane_value(scand != 0x7fffffff, scand, 0x7fffffff);
    if (s == 0x7fffffff || s >= n) {  // rounding left no row to claim x: no more candidates
      for (int jj = j + lane; jj < B; jj += 64) cand[jj] = -1;
      break;
    }
    // the lane holding row s records its interval [C_{s-1}, C_s) of the running sum
    const int owner = (s - r0) / RPT, loc = s - r0 - owner * RPT;
    double lo = base, ms = 0.0;
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      if (e < loc) lo += pm[e];
      if (e == loc) ms = pm[e];
    }
    const double flo = lane_d(lo, owner), fm = lane_d(ms, owner);
    if (lane == 0) cand[j] = s;
    // insert into the index-ordered list: lanes at and past the new position move up by one
    const int pos = __popcll(__ballot(lane < nd && c_idx < s));
    const int up_idx = __shfl_up(c_idx, 1, 64);
    const double up_lo = __shfl_up(c_lo, 1, 64), up_m = __shfl_up(c_m, 1, 64);
    if (lane == pos) {
      c_idx = s; c_lo = flo; c_m = fm;
    } else if (lane > pos) {
      c_idx = up_idx; c_lo = up_lo; c_m = up_m;
    }
    removed += fm;
    ++nd;
  }
}

// One thread per row (256 rows per workgroup): the candidate keys and, chunk by chunk, the
// candidate rows of F sit in LDS; F is read once, column by column (coalesced).
template <typename T, int D, int B>
__global__ void __launch_bounds__(NT) blk_column_kernel(BlockRpcArgs A) {
  __shared__ __attribute__((aligned(16))) float sKS[D][B];
  __shared__ __attribute__((aligned(16))) float sFS[64][B];
  __shared__ int sC[B];
  const StreamRpcArgs& a = A.s;
  const int h = blockIdx.y, tid = threadIdx.x, n = a.n;
  if (blk_done(A, h) || A.cand[(size_t)h * B] < 0) return;
  const int f0 = a.rank[h];
  const int i = blockIdx.x * NT + tid;
  const T* K = reinterpret_cast<const T*>(a.K) + (size_t)h * n * D;
  const float* F = a.F + (size_t)h * a.r * n;
  if (tid < B) sC[tid] = A.cand[(size_t)h * B + tid];
  __syncthreads();
  for (int e = tid; e < D * B; e += NT) {
    const int jj = e / D, ee = e % D, sj = sC[jj];
    sKS[ee][jj] = sj >= 0 ? ld_elem<T>(K + (size_t)sj * D + ee) : 0.f;
  }
  float acc[B];
#pragma unroll
  for (int jj = 0; jj < B; ++jj) acc[jj] = 0.f;
  for (int c0 = 0; c0 < f0; c0 += 64) {
    const int cc = min(64, f0 - c0);
    __syncthreads();
    for (int e = tid; e < cc * B; e += NT) {
      const int c = e / B, jj = e % B, sj = sC[jj];
      sFS[c][jj] = sj >= 0 ? F[(size_t)(c0 + c) * n + sj] : 0.f;
    }
    __syncthreads();
    if (i < n) {
      for (int c = 0; c < cc; ++c) {
        const float f = F[(size_t)(c0 + c) * n + i];
#pragma unroll
        for (int jj = 0; jj < B; jj += 4) {
          const float4 q = *reinterpret_cast<const float4*>(&sFS[c][jj]);
          acc[jj] = fmaf(f, q.x, acc[jj]); acc[jj + 1] = fmaf(f, q.y, acc[jj + 1]);
          acc[jj + 2] = fmaf(f, q.z, acc[jj + 2]); acc[jj + 3] = fmaf(f, q.w, acc[jj + 3]);
        }
      }
    }
  }
  __syncthreads();
  if (i >= n) return;
  float hk[B];
#pragma unroll
  for (int jj = 0; jj < B; ++jj) hk[jj] = 0.f;
  const T* kr = K + (size_t)i * D;
  for (int e = 0; e < D; ++e) {
    const float x = ld_elem<T>(kr + e);
#pragma unroll
    for (int jj = 0; jj < B; jj += 4) {
      const float4 q = *reinterpret_cast<const float4*>(&sKS[e][jj]);
      hk[jj] = fmaf(x, q.x, hk[jj]); hk[jj + 1] = fmaf(x, q.y, hk[jj + 1]);
      hk[jj + 2] = fmaf(x, q.z, hk[jj + 2]); hk[jj + 3] = fmaf(x, q.w, hk[jj + 3]);
    }
  }
  float* G = A.G + (size_t)h * B * n;
#pragma unroll
  for (int jj = 0; jj < B; ++jj) G[(size_t)jj * n + i] = __builtin_amdgcn_exp2f(hk[jj] * a.beta_log2e) - acc[jj];
}

// The factor rows at the round's candidates, negated, -F[S, :f0], into FS [f0][b] (by factor
// column), so that the column kernel reads them with coalesced loads and accumulates them onto
// the exponentials as they are.  Grid (blocks of 256 entries, heads).
template <int B>
__global__ void __launch_bounds__(256) blk_gather_kernel(BlockRpcArgs A) {
  const StreamRpcArgs& a = A.s;
  const int h = blockIdx.y;
  if (blk_done(A, h) || A.cand[(size_t)h * B] < 0) return;
  const int f0 = a.rank[h];
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= f0 * B) return;
  const int c = e / B, jj = e % B, sj = A.cand[(size_t)h * B + jj];
  A.FS[(size_t)h * a.r * B + e] = sj >= 0 ? -a.F[((size_t)h * a.r + c) * a.n + sj] : 0.f;
}

// The same candidate columns for bf16 keys on the matrix cores.  A workgroup takes 128 rows (32
// per wave); the candidates are the M dimension and the rows the N dimension of 32 x 32 tiles,
// so that a lane holds one row and every store of G is 32 consecutive rows.
//   kernel part: bf16 MFMAs, candidate keys from LDS, the wave's own key rows straight from
//                memory (the products of bf16 values are exact, the sums fp32);
//   exp2 in place, then the factor part on fp32 MFMAs (32 x 32 x 2): the candidates' factor
//   rows (gathered for the round by blk_gather_kernel), negated, and the rows' factor columns,
//   both read straight from memory, accumulated onto the exponentials.
template <int D, int B>
__global__ void __launch_bounds__(256) blk_column_mfma_kernel(BlockRpcArgs A) {
  constexpr int NC = (B + 31) / 32, BP = 32 * NC;  // candidate tiles (16 candidates use half of one)
  constexpr int KP = D + 8;                         // padded candidate-key row (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t sKS[BP * KP];
  __shared__ int sC[BP];
  const StreamRpcArgs& a = A.s;
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int n = a.n;
  if (blk_done(A, h) || A.cand[(size_t)h * B] < 0) return;
  const int f0 = a.rank[h];
  const int row = blockIdx.x * 128 + (tid >> 6) * 32 + l32;
  const bool rv = row < n;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.K) + (size_t)h * n * D;
  const float* F = a.F + (size_t)h * a.r * n;
  if (tid < BP) sC[tid] = tid < B ? A.cand[(size_t)h * B + tid] : -1;
  // the wave's key rows, requested before the staging barrier
  bf16x8 kb[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (rv) kb[kk] = *reinterpret_cast<const bf16x8*>(K + (size_t)row * D + 16 * kk + 8 * g);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) kb[kk][e] = (__bf16)0.f;
  }
  __syncthreads();
  for (int e = tid; e < BP * D / 8; e += 256) {
    const int jj = e / (D / 8), q = e % (D / 8), sj = sC[jj];
    const uint4 v = sj >= 0 ? reinterpret_cast<const uint4*>(K + (size_t)sj * D)[q] : uint4{0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(sKS + jj * KP + 8 * q) = v;
  }
  __syncthreads();
  f32x16 acc[NC];
#pragma unroll
  for (int t = 0; t < NC; ++t) acc[t] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int t = 0; t < NC; ++t)
      acc[t] = mfma32(*reinterpret_cast<const bf16x8*>(sKS + (32 * t + l32) * KP + 16 * kk + 8 * g), kb[kk], acc[t]);
  const float bl2e = a.beta_log2e;
#pragma unroll
  for (int t = 0; t < NC; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = __builtin_amdgcn_exp2f(acc[t][v] * bl2e);
  // factor part: 16 factor columns per batch; the candidates' rows from FS and this lane's
  // row from F, both coalesced, no LDS and no barrier
  // Loads use clamped indices and no conditions (a masked load compiles to a branch and a wait
  // per load); factor columns past f0 are zeroed afterwards, and the lanes of rows past n or of
  // candidate slots past b feed only outputs that are never stored.
  const float* FSh = A.FS + (size_t)h * a.r * B;
  const int rowc = rv ? row : n - 1;
  int jc[NC];  // candidate slot of each tile's lane, clamped into [0, b)
#pragma unroll
  for (int t = 0; t < NC; ++t) jc[t] = 32 * t + l32 < B ? 32 * t + l32 : 0;
  // Three register buffers rotate: a batch's products are issued after the loads of the batch
  // two ahead (the last batches load clamped, unused copies), so each wave keeps two batches of
  // loads in flight behind its matrix-core work.
  float fa0[8][NC], fb0[8], fa1[8][NC], fb1[8], fa2[8][NC], fb2[8];
  auto load_batch = [&](int c, float (&xa)[8][NC], float (&xb)[8]) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int ck = min(c + 2 * m + g, f0 - 1);
      xb[m] = F[(size_t)ck * n + rowc];
#pragma unroll
      for (int t = 0; t < NC; ++t) xa[m][t] = FSh[(size_t)ck * B + jc[t]];
    }
  };
  auto products = [&](int c, float (&xa)[8][NC], float (&xb)[8]) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
      if (c + 2 * m + g >= f0) xb[m] = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int t = 0; t < NC; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[m][t], xb[m], acc[t], 0, 0, 0);
  };
  if (f0 > 0) {
    load_batch(0, fa0, fb0);
    load_batch(16, fa1, fb1);
  }
  for (int c = 0; c < f0; c += 48) {
    load_batch(c + 32, fa2, fb2);
    __builtin_amdgcn_sched_barrier(0);
    products(c, fa0, fb0);
    if (c + 16 >= f0) break;
    load_batch(c + 48, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    products(c + 16, fa1, fb1);
    if (c + 32 >= f0) break;
    load_batch(c + 64, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    products(c + 32, fa2, fb2);
  }
  if (!rv) return;
  float* G = A.G + (size_t)h * B * n;
#pragma unroll
  for (int t = 0; t < NC; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int jj = 32 * t + 8 * (v >> 2) + 4 * g + (v & 3);
      if (jj < B) G[(size_t)jj * n + row] = acc[t][v];
    }
}

template <typename T, int D, int B>
__global__ void __launch_bounds__(4 * B) blk_factor_kernel(BlockRpcArgs A, int k) {
  constexpr int P = B + 4;
  __shared__ __attribute__((aligned(16))) float sA[B * P];
  __shared__ __attribute__((aligned(16))) float sCol[2][B];
  __shared__ __attribute__((aligned(16))) float sRow[2][B];
  __shared__ float sHd[B];
  __shared__ int sC[B];
  const StreamRpcArgs& a = A.s;
  const int h = blockIdx.x, tid = threadIdx.x, n = a.n;
  if (blk_done(A, h)) return;
  if (A.cand[(size_t)h * B] < 0) {  // no mass left: the loop stops
    if (tid == 0) a.flags[h] |= WC_DFLAG_BREAKDOWN;
    return;
  }
  const T* K = reinterpret_cast<const T*>(a.K) + (size_t)h * n * D;
  if (tid < B) {
    const int sj = A.cand[(size_t)h * B + tid];
    sC[tid] = sj;
    // kernel diagonal at the candidate, the scale of the leave-out test
    float q = 0.f;
    if (sj >= 0)
      for (int e = 0; e < D; ++e) {
        const float x = ld_elem<T>(K + (size_t)sj * D + e);
        q = fmaf(x, x, q);
      }
    sHd[tid] = sj >= 0 ? __builtin_amdgcn_exp2f(q * a.beta_log2e) : 0.f;
  }
  __syncthreads();
  const float* G = A.G + (size_t)h * B * n;
  for (int e = tid; e < B * B; e += 4 * B) {
    const int ii = e / B, jj = e % B, si = sC[ii];
    sA[ii * P + jj] = si >= 0 ? G[(size_t)jj * n + si] : 0.f;
  }
  __syncthreads();
  float* M = A.M + (size_t)h * B * B;
  elim_block<B, P>(sA, sHd, A.tol, sCol, sRow);
  store_block<B, P>(sA, M);
  if (tid == 0) {
    // kept candidates take the next free slots in order; once the slots are full the rest of
    // the round is dropped (later candidates were eliminated only against earlier ones)
    const int f0 = a.rank[h];
    int f = f0;
    for (int jj = 0; jj < B; ++jj) {
      int sl = -1;
      if (f < a.r && sA[jj * P + jj] > 0.f) {
        sl = f++;
        a.pivots[(size_t)h * a.r + sl] = sC[jj];
      }
      A.slot[(size_t)h * B + jj] = sl;
    }
    a.rank[h] = f;
    A.rounds[h] = k + 1;
  }
}

// New columns of F, residual update and block masses; `rows` rows per workgroup as the
// streaming loop, so that the masses line up with the blocks the sampler reads.
template <int B>
__global__ void __launch_bounds__(NT) blk_apply_kernel(BlockRpcArgs A, int k) {
  __shared__ __attribute__((aligned(16))) float sM[B][B];  // sM[jj][c] = M[jj][c]
  __shared__ int sSl[B], sP[B];
  __shared__ double red[NW];
  const StreamRpcArgs& a = A.s;
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, n = a.n;
  if ((a.flags[h] & WC_DFLAG_BREAKDOWN) || A.rounds[h] != k + 1) return;  // this round did not run
  const float* dg_in = ((k & 1) ? a.diag1 : a.diag0) + (size_t)h * n;
  float* dg_out = ((k & 1) ? a.diag0 : a.diag1) + (size_t)h * n;
  double* part_out = (k & 1) ? a.part0 : a.part1;
  const float* M = A.M + (size_t)h * B * B;
  for (int e = tid; e < B * B; e += NT) sM[e / B][e % B] = M[e];
  if (tid < B) {
    const int sl = A.slot[(size_t)h * B + tid];
    sSl[tid] = sl;
    sP[tid] = sl >= 0 ? A.cand[(size_t)h * B + tid] : -1;
  }
  __syncthreads();
  const float* G = A.G + (size_t)h * B * n;
  float* F = a.F + (size_t)h * a.r * n;
  double mass = 0.0;
  for (int i = b * a.rows + tid; i < min(n, (b + 1) * a.rows); i += NT) {
    float g[B];
#pragma unroll
    for (int c = 0; c < B; ++c) g[c] = G[(size_t)c * n + i];
    float dsum = 0.f;
    bool piv = false;
#pragma unroll 4
    for (int jj = 0; jj < B; ++jj) {
      const int sl = sSl[jj];
      if (sl < 0) continue;
      float f = 0.f;
#pragma unroll
      for (int c = 0; c < B; c += 4) {  // row jj of M, four entries per LDS read (broadcast)
        const float4 m4 = *reinterpret_cast<const float4*>(&sM[jj][c]);
        f = fmaf(g[c], m4.x, f);
        f = fmaf(g[c + 1], m4.y, f);
        f = fmaf(g[c + 2], m4.z, f);
        f = fmaf(g[c + 3], m4.w, f);
      }
      F[(size_t)sl * n + i] = f;
      dsum = fmaf(f, f, dsum);
      piv |= sP[jj] == i;
    }
    const float d = piv ? 0.f : dg_in[i] - dsum;
    dg_out[i] = d;
    mass += mass_of(d);
  }
  const double tot = block_sum(mass, red);
  if (tid == 0) part_out[(size_t)h * a.nblk + b] = tot;
}

// After the last round: a head with slots left over breaks down (empty slots, zero columns of
// F); a full one gets the trace after its last round; the final residual if asked for.
__global__ void __launch_bounds__(NT) blk_final_kernel(BlockRpcArgs A) {
  __shared__ double red[NW];
  const StreamRpcArgs& a = A.s;
  const int h = blockIdx.x, tid = threadIdx.x, n = a.n, nblk = a.nblk;
  const int rk = a.rank[h], kr = A.rounds[h];
  const double* part = (kr & 1) ? a.part1 : a.part0;
  const float* dg = ((kr & 1) ? a.diag1 : a.diag0) + (size_t)h * n;
  if (rk == a.r) {
    if (a.trace) {
      const int per = (nblk + NT - 1) / NT;
      double mine = 0.0;
      for (int e = 0; e < per; ++e) {
        const int bb = tid * per + e;
        if (bb < nblk) mine += part[(size_t)h * nblk + bb];
      }
      double T;
      block_excl_scan(mine, red, &T);
      if (tid == 0) a.trace[(size_t)h * (a.r + 1) + a.r] = T;
    }
  } else {
    if (tid == 0) a.flags[h] |= WC_DFLAG_BREAKDOWN;
    for (int t = rk + tid; t < a.r; t += NT) a.pivots[(size_t)h * a.r + t] = -1;
    for (size_t e = (size_t)rk * n + tid; e < (size_t)a.r * n; e += NT) a.F[(size_t)h * a.r * n + e] = 0.f;
  }
  if (a.diag_out)
    for (int i = tid; i < n; i += NT) a.diag_out[(size_t)h * n + i] = dg[i];
}

template <typename T, int D, int B>
static hipError_t run_block(BlockRpcArgs A, hipStream_t st) {
  StreamRpcArgs& a = A.s;
  const dim3 grid(a.nblk, a.H);
  hipError_t e;
  if (!a.u_forced) {
    const size_t nu = (size_t)a.H * kBlockDraws * a.r;
    hipLaunchKernelGGL(blk_uniforms_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, st, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((rpc_init_kernel<T, D>), grid, dim3(NT), 0, st, a, a.rows);
  hipLaunchKernelGGL(blk_init_kernel, dim3(a.H), dim3(NT), 0, st, A);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t lds = 2 * (size_t)a.nblk * sizeof(double);
  const bool wide = a.rows == 1024;  // rows per block: 1024 (16 per lane) or 256 (4 per lane)
  const bool resident = wide && a.nblk <= 2;  // the sub-head's rows in registers (2048 rows at most)
  if (lds > 48 * 1024) {
    const void* fn = wide ? reinterpret_cast<const void*>(&blk_sample_kernel<16, 0>)
                          : reinterpret_cast<const void*>(&blk_sample_kernel<4, 0>);
    if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess) return e;
  }
  const int colgrid = (a.n + NT - 1) / NT;
  const int rounds = kBlockDraws * a.r / B;
  for (int k = 0; k < rounds; ++k) {
    if (resident) hipLaunchKernelGGL((blk_sample_kernel<16, 2>), dim3(a.H), dim3(64), lds, st, A, k);
    else if (wide) hipLaunchKernelGGL((blk_sample_kernel<16, 0>), dim3(a.H), dim3(64), lds, st, A, k);
    else hipLaunchKernelGGL((blk_sample_kernel<4, 0>), dim3(a.H), dim3(64), lds, st, A, k);
    if constexpr (sizeof(T) == 2) {
      hipLaunchKernelGGL((blk_gather_kernel<B>), dim3((a.r * B + 255) / 256, a.H), dim3(256), 0, st, A);
      hipLaunchKernelGGL((blk_column_mfma_kernel<D, B>), dim3((a.n + 127) / 128, a.H), dim3(256), 0, st, A);
    }
    else
      hipLaunchKernelGGL((blk_column_kernel<T, D, B>), dim3(colgrid, a.H), dim3(NT), 0, st, A);
    hipLaunchKernelGGL((blk_factor_kernel<T, D, B>), dim3(a.H), dim3(4 * B), 0, st, A, k);
    hipLaunchKernelGGL((blk_apply_kernel<B>), grid, dim3(NT), 0, st, A, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(blk_final_kernel, dim3(a.H), dim3(NT), 0, st, A);
  return hipGetLastError();
}

template <int B>
static hipError_t run_block_b(const BlockRpcArgs& A, hipStream_t st) {
  const StreamRpcArgs& a = A.s;
  if (a.bf16) return a.d == 64 ? run_block<uint16_t, 64, B>(A, st) : run_block<uint16_t, 128, B>(A, st);
  return a.d == 64 ? run_block<float, 64, B>(A, st) : run_block<float, 128, B>(A, st);
}

hipError_t launch_rpc_block(const BlockRpcArgs& A, hipStream_t st) {
  switch (A.b) {
    case 16: return run_block_b<16>(A, st);
    case 32: return run_block_b<32>(A, st);
    case 64: return run_block_b<64>(A, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rpc_stream(const StreamRpcArgs& a, hipStream_t st) {
  const int rows = a.rows;
  if (a.bf16) return a.d == 64 ? run_rpc<uint16_t, 64>(a, rows, st) : run_rpc<uint16_t, 128>(a, rows, st);
  return a.d == 64 ? run_rpc<float, 64>(a, rows, st) : run_rpc<float, 128>(a, rows, st);
}

}  // namespace wc
