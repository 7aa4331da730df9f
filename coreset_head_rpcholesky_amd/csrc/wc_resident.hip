// Resident WildCat forward: one workgroup per head, the whole head on one CU.
//
// For short heads (n <= 256 keys, bf16 inputs, r <= 32) every row of K and of the partial
// Cholesky factor F lives in the registers of the thread that owns the row, so the r
// sequential pivot steps of randomly pivoted Cholesky (gist.science/de/paper/2602.10056,
// "Methodik" part 1) run with two workgroup barriers each and no memory traffic beyond the
// compulsory reads of Q, K, V and the write of O.  The Nystroem weights ("Methodik" part 2)
// and the attention over the coreset follow in the same launch on the bf16 matrix cores.
//
// Per step t (identical arithmetic in every thread, so every thread agrees):
//   mass p_i = max(diag_i, 0) -> wave inclusive scan (fp64) -> wave totals in LDS (barrier)
//   T = sum of wave totals in wave order; s = min{i : C_i > u_t T} (first wave whose running
//   total exceeds u_t T, then the first lane in it); the thread owning row s publishes k_s,
//   F[s, :t] and g_s = H_ss - |F[s, :t]|^2 (barrier); every thread then forms
//   g_i = exp(beta k_i.k_s) - F[i, :t].F[s, :t], F[i, t] = g_i / sqrt(g_s), diag_i -= F[i, t]^2.
#include "wc_device.h"
#include "wc_kernels.h"

#include <type_traits>

namespace wc {

template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_d(double x, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
  return __hiloint2double(hi, lo);
}
// Inclusive fp64 scan over the wave: row_shr within 16-lane rows, then row offsets.
__device__ __forceinline__ double wave_scan_fast(double x) {
  x += dpp_d<0x111>(x);
  x += dpp_d<0x112>(x);
  x += dpp_d<0x114>(x);
  x += dpp_d<0x118>(x);
  const double r0 = readlane_d(x, 15), r1 = readlane_d(x, 31), r2 = readlane_d(x, 47);
  const double o2 = r0 + r1, o3 = o2 + r2;
  const int row = (threadIdx.x & 63) >> 4;
  if (row == 1) x += r0;
  if (row == 2) x += o2;
  if (row == 3) x += o3;
  return x;
}

// dot(k_a, k_b) of two keys held as packed bf16 pairs; fixed association order.
template <int D2, typename PA, typename PB>
__device__ __forceinline__ float dot_bf16(const PA& a, const PB& b) {
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int q = 0; q < D2; q += 2) {
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a[q]),
                                           __builtin_bit_cast(bf16x2, b[q]), acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a[q + 1]),
                                           __builtin_bit_cast(bf16x2, b[q + 1]), acc1, false);
  }
  return acc0 + acc1;
}

// sum_{j < T} a[j] b[j] with a fixed association order (two interleaved chains).
template <int T, typename PA, typename PB>
__device__ __forceinline__ float dot_prefix(const PA& a, const PB& b) {
  float c0 = 0.f, c1 = 0.f;
#pragma unroll
  for (int j = 0; j + 1 < T; j += 2) {
    c0 = fmaf(a[j], b[j], c0);
    c1 = fmaf(a[j + 1], b[j + 1], c1);
  }
  if (T & 1) c0 = fmaf(a[T - 1], b[T - 1], c0);
  return c0 + c1;
}

template <int I, int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>{});
    static_for<I + 1, N>(fn);
  }
}

// Position of coreset index j inside a permuted 32-chunk, so that the accumulator layout
// of the score MFMA feeds the value MFMA directly (see the attention phase below).
__device__ __forceinline__ int perm32(int j) {
  const int jb = j & ~31, jj = j & 31;
  const int qq = jj >> 4, rem = jj & 15;
  const int g = (rem & 7) >> 2, e = ((rem >> 3) << 2) | (rem & 3);
  return jb + 16 * qq + 8 * g + e;
}

template <int D, int DV, int R, int NT>
struct ResidentSmem {
  static constexpr int NW = NT / 64;
  static constexpr int CH = ((4 * R + 2 * DV) * 128 <= 32768 && NT >= 128) ? 128 : 64;
  static constexpr int KSP = D + 8;   // padded row length of the staged coreset keys (bf16)
  static constexpr int WPP = R + 8;   // padded row length of the permuted weights (bf16)
  static constexpr int XP = DV + 1;   // row length of X (fp32)
  // phase-2 staging (aliased with X after the chunk loop)
  static constexpr int STAGE_BYTES = (2 * R * CH + DV * CH) * 2;
  static constexpr int X_BYTES = R * XP * 4;
  static constexpr int A_BYTES = STAGE_BYTES > X_BYTES ? STAGE_BYTES : X_BYTES;
};

template <int D, int DV, int R, int NT>
__global__ void __launch_bounds__(NT) resident_kernel(ResidentArgs a) {
  using S = ResidentSmem<D, DV, R, NT>;
  constexpr int NW = S::NW, D2 = D / 2, CH = S::CH;
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int n = a.n, r = a.r;
  const bool valid = tid < n;

  __shared__ double s_wsum[NW];
  __shared__ int s_piv;
  __shared__ float s_gs, s_rs;
  __shared__ float s_u[R];
  __shared__ uint32_t s_flag;
  __shared__ __attribute__((aligned(16))) uint32_t s_ks[D2];
  __shared__ __attribute__((aligned(16))) float s_fs[R];
  __shared__ float s_L[R][R + 1];
  __shared__ int s_pivots[R];
  __shared__ __attribute__((aligned(16))) unsigned char s_A[S::A_BYTES];
  __shared__ __attribute__((aligned(16))) __bf16 s_Ks[R * S::KSP];
  __shared__ __attribute__((aligned(16))) __bf16 s_Wp[DV * S::WPP];
  __shared__ float s_Wden[R];

  // ---------------- load own key row ----------------
  uint32_t kr[D2];
  const uint16_t* Kh = a.K + (size_t)h * n * D;
  if (valid) {
    const uint4* src = reinterpret_cast<const uint4*>(Kh + (size_t)tid * D);
#pragma unroll
    for (int q = 0; q < D / 8; ++q) {
      const uint4 v = src[q];
      kr[4 * q] = v.x; kr[4 * q + 1] = v.y; kr[4 * q + 2] = v.z; kr[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < D2; ++q) kr[q] = 0u;
  }
  const float bl2e = a.beta_log2e;
  const float d0 = valid ? __builtin_amdgcn_exp2f(dot_bf16<D2>(kr, kr) * bl2e) : 0.f;
  float dg = d0;
  float fr[R];
#pragma unroll
  for (int j = 0; j < R; ++j) fr[j] = 0.f;
  if (tid == 0) {
    s_flag = 0u;
    s_piv = -1;
  }
  // the r pivot uniforms, drawn once (first use is after the first barrier)
  if (tid < r) s_u[tid] = pivot_uniform(a.u_forced, a.seed, h, r, tid);
  int rk = r;
  uint32_t flg = 0u;

  // ---------------- randomly pivoted Cholesky ----------------
  bool alive = true;
  static_for<0, R>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    if (!alive || t >= r) return;
    const double pd = valid ? mass_of(dg) : 0.0;
    const double x = wave_scan_fast(pd);
    if (lane == 63) s_wsum[wid] = x;
    __syncthreads();
    double T = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) T += s_wsum[w];
    if (tid == 0 && a.trace) a.trace[(size_t)h * (r + 1) + t] = __builtin_isfinite(T) ? T : 0.0;
    if (!(T > 0.0) || !__builtin_isfinite(T)) {
      rk = t;
      flg |= WC_DFLAG_BREAKDOWN | (__builtin_isfinite(T) ? 0u : WC_DFLAG_NONFINITE);
      alive = false;
      return;
    }
    const double uT = (double)s_u[t] * T;
    double acc = 0.0, pre = 0.0;
    int wstar = -1, wlast = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const double tw = s_wsum[w];
      const double nxt = acc + tw;
      if (w == wid) pre = acc;
      if (wstar < 0 && nxt > uT) wstar = w;
      if (tw > 0.0) wlast = w;
      acc = nxt;
    }
    bool winner = false;
    if (wstar >= 0) {
      const uint64_t b = ballot(pre + x > uT);
      if (wid == wstar) winner = lane == __builtin_ctzll(b);
    } else {  // u T rounded onto the total: last row with positive mass
      const uint64_t b = ballot(pd > 0.0);
      if (wid == wlast) winner = lane == 63 - __builtin_clzll(b);
    }
    if (winner) {
      s_piv = tid;
      const float g = d0 - dot_prefix<t>(fr, fr);
      s_gs = g;
      s_rs = 1.0f / sqrtf(g);
#pragma unroll
      for (int q = 0; q < D2; ++q) s_ks[q] = kr[q];
#pragma unroll
      for (int j = 0; j < t; ++j) { s_fs[j] = fr[j]; s_L[t][j] = fr[j]; }
    }
    __syncthreads();
    const int s = s_piv;
    const float gs = s_gs;
    if (s < 0 || s >= n) {  // no row claimed the draw: cannot happen for finite T > 0
      rk = t;
      flg |= WC_DFLAG_BREAKDOWN | WC_DFLAG_NONFINITE;
      alive = false;
      return;
    }
    if (tid == 0) {
      s_pivots[t] = s;
      if (a.pivots) a.pivots[(size_t)h * r + t] = s;
    }
    if (!(gs > 0.f) || !__builtin_isfinite(gs)) {
      rk = t;
      flg |= WC_DFLAG_BREAKDOWN | (__builtin_isfinite(gs) ? 0u : WC_DFLAG_NONFINITE);
      alive = false;
      return;
    }
    const float rs = s_rs;
    const float hcol = __builtin_amdgcn_exp2f(dot_bf16<D2>(kr, s_ks) * bl2e);
    const float gi = hcol - dot_prefix<t>(fr, s_fs);
    const float f = valid ? gi * rs : 0.f;
    fr[t] = f;
    dg = (tid == s) ? 0.f : dg - f * f;
    if (tid == s) s_L[t][t] = f;
  });

  // trace after the last step (reported only when all r steps completed)
  if (a.trace && rk == r) {
    const double pd = valid ? mass_of(dg) : 0.0;
    const double x = wave_scan_fast(pd);
    __syncthreads();
    if (lane == 63) s_wsum[wid] = x;
    __syncthreads();
    double T = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) T += s_wsum[w];
    if (tid == 0) a.trace[(size_t)h * (r + 1) + r] = T;
  }
  if (tid == 0) {
    a.rank[h] = rk;
    a.flags[h] = flg;
    if (a.trace)
      for (int t = rk + 1; t <= r; ++t) a.trace[(size_t)h * (r + 1) + t] = 0.0;
    if (a.pivots)
      for (int t = rk; t < r; ++t) a.pivots[(size_t)h * r + t] = -1;
  }
  if (a.F && valid) {
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j < r) a.F[((size_t)h * r + j) * n + tid] = fr[j];
  }
  if (a.diag && valid) a.diag[(size_t)h * n + tid] = dg;
  if (!a.O) return;  // pivot loop only

  // ---------------- Nystroem weights: X = F^T [V, 1], W = L^{-T} X ----------------
  // X tiles (32 x 32) on the bf16 matrix cores; F enters as hi + lo bf16 parts, V is exact
  // in bf16.  Tile list: (jt, ct) for ct < DV/32 plus one "ones" tile per jt whose first
  // column is the column sum of F (the normaliser column of X).
  constexpr int NJT = R / 32, NCT = DV / 32, NTILES = NJT * (NCT + 1);
  constexpr int TPW = (NTILES + NW - 1) / NW;
  __bf16* FtH = reinterpret_cast<__bf16*>(s_A);           // [R][CH]
  __bf16* FtL = FtH + R * CH;                              // [R][CH]
  __bf16* Vt = FtL + R * CH;                               // [DV][CH]
  f32x16 acc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[k][v] = 0.f;
  const uint16_t* Vh = a.V + (size_t)h * n * DV;
  for (int c0 = 0; c0 < NT; c0 += CH) {
    __syncthreads();
    if (tid >= c0 && tid < c0 + CH) {
      const int ii = tid - c0;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        __bf16 hi, lo;
        split_bf16(fr[j], hi, lo);
        FtH[j * CH + ii] = hi;
        FtL[j * CH + ii] = lo;
      }
      if (valid) {
        const uint4* src = reinterpret_cast<const uint4*>(Vh + (size_t)tid * DV);
#pragma unroll
        for (int q = 0; q < DV / 8; ++q) {
          const uint4 v = src[q];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            Vt[(8 * q + 2 * e) * CH + ii] = __builtin_bit_cast(__bf16, (uint16_t)(w4[e] & 0xffffu));
            Vt[(8 * q + 2 * e + 1) * CH + ii] = __builtin_bit_cast(__bf16, (uint16_t)(w4[e] >> 16));
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < DV; ++c) Vt[c * CH + ii] = (__bf16)0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int tile = wid + k * NW;
      if (tile < NTILES) {
        const int jt = tile / (NCT + 1), ct = tile % (NCT + 1);
        for (int kk = 0; kk < CH; kk += 16) {
          const int off = (jt * 32 + l32) * CH + kk + 8 * g;
          const bf16x8 ah = *reinterpret_cast<const bf16x8*>(FtH + off);
          const bf16x8 al = *reinterpret_cast<const bf16x8*>(FtL + off);
          bf16x8 b;
          if (ct < NCT) {
            b = *reinterpret_cast<const bf16x8*>(Vt + (ct * 32 + l32) * CH + kk + 8 * g);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = (__bf16)1.0f;
          }
          acc[k] = mfma32(ah, b, acc[k]);
          acc[k] = mfma32(al, b, acc[k]);
        }
      }
    }
  }
  __syncthreads();
  float* Xs = reinterpret_cast<float*>(s_A);  // [R][DV+1]
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int tile = wid + k * NW;
    if (tile < NTILES) {
      const int jt = tile / (NCT + 1), ct = tile % (NCT + 1);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = jt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        if (ct < NCT) Xs[j * S::XP + ct * 32 + l32] = acc[k][v];
        else if (l32 == 0) Xs[j * S::XP + DV] = acc[k][v];
      }
    }
  }
  __syncthreads();
  // backward substitution L^T W = X, one column per thread
  for (int c = tid; c <= DV; c += NT) {
    float xv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) xv[j] = Xs[j * S::XP + c];
#pragma unroll
    for (int t = R - 1; t >= 0; --t) {
      float w = 0.f;
      if (t < rk) {
        w = xv[t] / s_L[t][t];
#pragma unroll
        for (int j = 0; j < t; ++j) xv[j] = fmaf(-s_L[t][j], w, xv[j]);
      }
      if (a.W && t < r) a.W[((size_t)h * r + t) * (DV + 1) + c] = w;
      if (c < DV) s_Wp[c * S::WPP + perm32(t)] = (__bf16)w;
      else s_Wden[t] = w;
    }
  }
  // stage the coreset keys (bf16) for the score MFMA
  for (int e = tid; e < R * (D / 8); e += NT) {
    const int j = e / (D / 8), q = e % (D / 8);
    uint4 v = {0u, 0u, 0u, 0u};
    if (j < rk) v = reinterpret_cast<const uint4*>(Kh + (size_t)s_pivots[j] * D)[q];
    *reinterpret_cast<uint4*>(s_Ks + j * S::KSP + 8 * q) = v;
  }
  __syncthreads();

  // ---------------- attention over the weighted coreset ----------------
  // Per wave a tile of 32 queries.  Scores S^T = K_S Q^T (32 coreset x 32 queries) land in
  // the accumulator layout; exp of them is directly the B operand of Y^T = W^T P^T when the
  // coreset index inside each 32-chunk is permuted by perm32 on the W side.
  const uint16_t* Qh = a.Q + (size_t)h * a.m * D;
  uint16_t* Oh = a.O + (size_t)h * a.m * DV;
  const int m = a.m;
  bool bad = false;
  for (int qt = wid; qt * 32 < m; qt += NW) {
    const int q = qt * 32 + l32;
    const bool qv = q < m;
    bf16x8 qb[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (qv) qb[kk] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)q * D + 16 * kk + 8 * g);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[kk][e] = (__bf16)0.f;
    }
    f32x16 y[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) y[ct][v] = 0.f;
    float den = 0.f;
#pragma unroll
    for (int jb = 0; jb < R / 32; ++jb) {
      f32x16 sc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(s_Ks + (jb * 32 + l32) * S::KSP + 16 * kk + 8 * g);
        sc = mfma32(ak, qb[kk], sc);
      }
      bf16x8 pb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = jb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        const float p = (j < rk) ? __builtin_amdgcn_exp2f(sc[v] * bl2e) : 0.f;
        den = fmaf(p, s_Wden[j], den);
        pb[v >> 3][v & 7] = (__bf16)p;
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const bf16x8 aw = *reinterpret_cast<const bf16x8*>(s_Wp + (ct * 32 + l32) * S::WPP + jb * 32 + 16 * qq + 8 * g);
          y[ct] = mfma32(aw, pb[qq], y[ct]);
        }
    }
    den += __shfl_xor(den, 32, 64);
    if (qv) {
      bad |= !(den > 0.f);
      const float inv = 1.0f / den;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int c = ct * 32 + 8 * v4 + 4 * g;
          uint16_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(uint16_t, (__bf16)(y[ct][4 * v4 + e] * inv));
          uint2 pk;
          pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
          pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
          *reinterpret_cast<uint2*>(Oh + (size_t)q * DV + c) = pk;
        }
    }
  }
  if (bad) atomicOr(&s_flag, WC_DFLAG_DENOM);
  __syncthreads();
  if (tid == 0 && s_flag) a.flags[h] = flg | s_flag;
}

// This file is compiled once per (WC_RES_D, WC_RES_DV) pair so the instantiations build in
// parallel; each object exports launch_resident_<d>_<dv>.
#ifndef WC_RES_D
#define WC_RES_D 64
#endif
#ifndef WC_RES_DV
#define WC_RES_DV 64
#endif
#define WC_CAT_(a, b, c) a##b##_##c
#define WC_CAT(a, b, c) WC_CAT_(a, b, c)

hipError_t WC_CAT(launch_resident_, WC_RES_D, WC_RES_DV)(const ResidentArgs& a, int heads, hipStream_t st) {
  hipLaunchKernelGGL((resident_kernel<WC_RES_D, WC_RES_DV, kResidentR, kResidentThreads>), dim3(heads),
                     dim3(kResidentThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace wc
