// Resident WildCat forward: one workgroup per head, the whole head on one CU.
//
// For short heads (n <= 256 keys, bf16 inputs, r <= 32) the r sequential pivot steps of
// randomly pivoted Cholesky (gist.science/de/paper/2602.10056, "Methodik" part 1) run out of
// registers and LDS with one barrier per step and no memory traffic beyond the compulsory
// reads of Q, K, V and the write of O.  The Nystroem weights ("Methodik" part 2) and the
// attention over the coreset follow in the same launch on the bf16 matrix cores.
//
// Two waves per head; lane l of wave w owns the consecutive key rows a = 2(64w + l) and a + 1.
// Its keys and its rows of the factor F sit in registers; copies of the keys, of the rows of
// F (with the initial diagonal H_ii appended) and of the residual diagonal sit in LDS.  Step t,
// after the barrier that ends step t-1 (identical arithmetic in every thread, so every thread
// agrees without further communication):
//   T = w0 + w1, the two wave totals of the masses max(diag, 0) (fp64, each a wave scan over
//       the row pairs);
//   s = min{i : C_i > u_t T}: the wave whose running total first exceeds u_t T is searched by
//       ballot, from its own registers in that wave and from the residual diagonal in LDS
//       (re-scanned with the same arithmetic) in the other;
//   g_s = H_ss - |F[s, :t]|^2 from LDS, then every thread forms, for its two rows,
//   g_i = exp(beta k_i.k_s) - F[i, :t].F[s, :t], F[i, t] = g_i / sqrt(g_s), diag_i -= F[i, t]^2,
//   stores them to LDS, scans its wave's masses for step t+1 and meets the other wave at the
//   barrier.
#include "wc_device.h"
#include "wc_kernels.h"

#include <type_traits>

namespace wc {

// Lane movement of an fp64 value; lanes with no source lane read zero (bound_ctrl).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), CTRL, 0xf, 0xf, true);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_d(double x, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
  return __hiloint2double(hi, lo);
}
// Lane broadcast of an fp64 value into the rows of ROWMASK; the other rows read zero.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_rows_d(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), CTRL, ROWMASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), CTRL, ROWMASK, 0xf, false);
  return __hiloint2double(hi, lo);
}
// Two independent inclusive fp64 scans over the wave, level by level side by side (the step is
// latency-bound, so the two dependency chains overlap): row_shr within 16-lane rows, then the
// last lane of row 0 into row 1 and of row 2 into row 3 (row_bcast:15), then the last lane of
// row 1 into rows 2 and 3 (row_bcast:31).  Each scan adds in the same order as a scan of its
// own; rows that receive nothing add +0, which leaves their non-negative sums unchanged.
__device__ __forceinline__ void wave_scan2(double& x, double& y) {
  x += dpp_d<0x111>(x);
  y += dpp_d<0x111>(y);
  x += dpp_d<0x112>(x);
  y += dpp_d<0x112>(y);
  x += dpp_d<0x114>(x);
  y += dpp_d<0x114>(y);
  x += dpp_d<0x118>(x);
  y += dpp_d<0x118>(y);
  x += dpp_rows_d<0x142, 0xa>(x);
  y += dpp_rows_d<0x142, 0xa>(y);
  x += dpp_rows_d<0x143, 0xc>(x);
  y += dpp_rows_d<0x143, 0xc>(y);
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


// Position of coreset index j inside a permuted 32-chunk, so that the accumulator layout
// of the score MFMA feeds the value MFMA directly (see the attention phase below).
__device__ __forceinline__ int perm32(int j) {
  const int jb = j & ~31, jj = j & 31;
  const int qq = jj >> 4, rem = jj & 15;
  const int g = (rem & 7) >> 2, e = ((rem >> 3) << 2) | (rem & 3);
  return jb + 16 * qq + 8 * g + e;
}

// Dynamic LDS of the resident kernel.  During the pivot loop: the keys [n][D/2] (packed bf16
// pairs), the rows of F [n][R+1] (the last slot holds H_ii; R+1 is odd, so the column stores
// of one step spread over the banks) and the residual diagonal double-buffered [2][256].  After
// the loop the weights and attention buffers reuse the same bytes.
template <int D, int DV, int R, int NT>
struct ResidentSmem {
  static constexpr int NW = NT / 64;
  static constexpr int FS = R + 1;    // row stride of F in LDS
  static constexpr int CH = 128;      // rows per staging chunk of the weights GEMM
  static constexpr int KSP = D + 8;   // padded row length of the staged coreset keys (bf16)
  static constexpr int WPP = R + 8;   // padded row length of the permuted weights (bf16)
  static constexpr int XP = DV + 1;   // row length of X (fp32)
  // phase-2 staging (aliased with X after the chunk loop)
  static constexpr int STAGE_BYTES = (2 * R * CH + DV * CH) * 2;
  static constexpr int X_BYTES = R * XP * 4;
  static constexpr int A_BYTES = STAGE_BYTES > X_BYTES ? STAGE_BYTES : X_BYTES;
  static constexpr int KS_OFF = A_BYTES;
  static constexpr int WP_OFF = KS_OFF + R * KSP * 2;
  static constexpr int WDEN_OFF = WP_OFF + DV * WPP * 2;
  static constexpr int L_OFF = WDEN_OFF + R * 4;
  static constexpr int LS = R + 4;    // row stride of L (16-byte rows; column R holds 1 / L_tt)
  static constexpr int P2_BYTES = L_OFF + R * LS * 4;
  static_assert(L_OFF % 16 == 0, "16-byte rows of L");
  // pivot-loop region, for n keys.  At n = 197 (d = 64) this region plus the kernel's ~270
  // bytes of static arrays just lets three workgroups share a CU; 256 more bytes of static LDS
  // were measured to drop that to two (1.5x slower at 768 heads).
  __host__ __device__ static constexpr int f_off(int n) { return n * D * 2; }
  static constexpr int DGS = 2 * NT;  // row stride of each residual-diagonal buffer (all rows)
  __host__ __device__ static constexpr int dg_off(int n) { return (f_off(n) + n * FS * 4 + 15) & ~15; }
  __host__ __device__ static constexpr int loop_bytes(int n) { return dg_off(n) + 2 * DGS * 4; }
  __host__ __device__ static constexpr int bytes(int n) {
    return loop_bytes(n) > P2_BYTES ? loop_bytes(n) : P2_BYTES;
  }
};

// Masses of a lane's row pair, their wave scan (pair sums), and the inclusive prefix of the
// first row of the pair: xa = x - m_b.
struct PairScan {
  double x, xa;
  bool pa, pb;  // rows with positive mass
};
// Both waves' row pairs at this lane position (rows 2l, 2l+1 and 128 + 2l, 128 + 2l + 1).
// Rows past the last key hold zero in both residual buffers.
__device__ __forceinline__ void pair_scan2(float2 d0, float2 d1, PairScan& q0, PairScan& q1) {
  const double m0a = mass_of(d0.x), m0b = mass_of(d0.y), m1a = mass_of(d1.x), m1b = mass_of(d1.y);
  double x0 = m0a + m0b, x1 = m1a + m1b;
  wave_scan2(x0, x1);
  q0 = {x0, x0 - m0b, m0a > 0.0, m0b > 0.0};
  q1 = {x1, x1 - m1b, m1a > 0.0, m1b > 0.0};
}

// d = dv = 64 keeps to 256 registers, so that two waves fit a SIMD and three workgroups a CU
// (the short heads run 768 at a time at n = 197).
template <int D, int DV, int R, int NT>
__global__ void __launch_bounds__(NT, (D == 64 && DV == 64) ? 2 : 1) resident_kernel(ResidentArgs a) {
  using S = ResidentSmem<D, DV, R, NT>;
  constexpr int NW = S::NW, D2 = D / 2, FS = S::FS, CH = S::CH, DGS = S::DGS;
  static_assert(NW == 2, "two waves per head");
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int n = a.n, r = a.r;
  const int ra = 2 * tid;                 // own rows ra, ra + 1
  const bool va = ra < n, vb = ra + 1 < n;

  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  __shared__ float s_u[R];
  __shared__ uint32_t s_flag;
  __shared__ int s_pivots[R];
  uint32_t* sK = reinterpret_cast<uint32_t*>(s_dyn);                 // [n][D2]
  float* sF = reinterpret_cast<float*>(s_dyn + S::f_off(n));         // [n][FS]
  float* sDg = reinterpret_cast<float*>(s_dyn + S::dg_off(n));       // [2][DGS]

  // ---------------- load own key rows ----------------
  uint32_t kr[2][D2];
  const uint16_t* Kh = a.K + (size_t)h * n * D;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = ra + p;
    if (row < n) {
      const uint4* src = reinterpret_cast<const uint4*>(Kh + (size_t)row * D);
#pragma unroll
      for (int q = 0; q < D / 8; ++q) {
        const uint4 v = src[q];
        kr[p][4 * q] = v.x; kr[p][4 * q + 1] = v.y; kr[p][4 * q + 2] = v.z; kr[p][4 * q + 3] = v.w;
        reinterpret_cast<uint4*>(sK + row * D2)[q] = v;
      }
    } else {
#pragma unroll
      for (int q = 0; q < D2; ++q) kr[p][q] = 0u;
    }
  }
  const float bl2e = a.beta_log2e;
  float dg[2], fr[2][R];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = ra + p;
    const float d0 = row < n ? __builtin_amdgcn_exp2f(dot_bf16<D2>(kr[p], kr[p]) * bl2e) : 0.f;
    dg[p] = d0;
#pragma unroll
    for (int j = 0; j < R; ++j) fr[p][j] = 0.f;
    if (row < n) sF[row * FS + R] = d0;
    sDg[row] = d0;          // zero past the last key, in both buffers
    sDg[DGS + row] = 0.f;
  }
  if (tid == 0) s_flag = 0u;
  // the r pivot uniforms, drawn once (first use is after the first barrier)
  if (tid < r) s_u[tid] = pivot_uniform(a.u_forced, a.seed, h, r, tid);
  __syncthreads();
  int rk = r;
  uint32_t flg = 0u;
  double T = 0.0;

  // ---------------- randomly pivoted Cholesky ----------------
  bool alive = true;
  static_for<0, R>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    constexpr int buf = t & 1;
    if (!alive || t >= r) return;
    // Both waves' row pairs at this lane position: scanned in two independent chains, so
    // every wave holds both wave totals and the prefix sums of whichever wave is crossed.
    const float2 d0p = reinterpret_cast<const float2*>(sDg + buf * DGS)[lane];
    const float2 d1p = reinterpret_cast<const float2*>(sDg + buf * DGS)[64 + lane];
    PairScan q0, q1;
    pair_scan2(d0p, d1p, q0, q1);
    const double w0 = readlane_d(q0.x, 63), w1 = readlane_d(q1.x, 63);
    T = w0 + w1;
    // Breakdown (T <= 0, no row claims the draw, g_s <= 0, anything non-finite) is collected
    // in one flag; the step's reads stay in bounds either way and its updates are skipped.
    const bool tfin = __builtin_isfinite(T);
    uint32_t bad = (T > 0.0 && tfin) ? 0u : (WC_DFLAG_BREAKDOWN | (tfin ? 0u : WC_DFLAG_NONFINITE));
    // the wave holding the crossing (or, if u T rounded onto the total, the last row with
    // positive mass), and the running total before it
    const double uT = (double)s_u[t] * T;
    const bool cross = T > uT;
    const int wsel = (w0 > uT || (!cross && !(w1 > 0.0))) ? 0 : 1;
    const double pre = wsel == 1 ? w0 : 0.0;
    const PairScan& q = wsel == 1 ? q1 : q0;
    const uint64_t bx = ballot(cross ? pre + q.x > uT : (q.pa || q.pb));
    const uint64_t bs = ballot(cross ? !(pre + q.xa > uT) : q.pb);  // second row of the pair
    const int L = cross ? (bx ? __builtin_ctzll(bx) : 0) : (bx ? 63 - __builtin_clzll(bx) : 0);
    int s = 2 * (64 * wsel + L) + (int)((bs >> L) & 1);
    if (!bx || s >= n) {  // no row claimed the draw: cannot happen for finite T > 0
      bad |= WC_DFLAG_BREAKDOWN | WC_DFLAG_NONFINITE;
      s = 0;
    }
    // pivot row of F, the pivot key and everything that needs only them, side by side
    const float* fsrow = sF + s * FS;
    float fs[t > 0 ? t : 1];
#pragma unroll
    for (int j = 0; j < t; ++j) fs[j] = fsrow[j];
    uint32_t ks[D2];
#pragma unroll
    for (int q4 = 0; q4 < D / 8; ++q4) {
      const uint4 v = reinterpret_cast<const uint4*>(sK + s * D2)[q4];
      ks[4 * q4] = v.x; ks[4 * q4 + 1] = v.y; ks[4 * q4 + 2] = v.z; ks[4 * q4 + 3] = v.w;
    }
    const float gs = fsrow[R] - dot_prefix<t>(fs, fs);
    float hk[2], corr[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      hk[p] = dot_bf16<D2>(kr[p], ks);
      corr[p] = dot_prefix<t>(fr[p], fs);
    }
    if (!bad && !(gs > 0.f && __builtin_isfinite(gs)))
      bad = WC_DFLAG_BREAKDOWN | (__builtin_isfinite(gs) ? 0u : WC_DFLAG_NONFINITE);
    if (tid == 0 && a.trace) a.trace[(size_t)h * (r + 1) + t] = tfin ? T : 0.0;
    if (bad) {
      rk = t;
      flg |= bad;
      alive = false;
      return;
    }
    if (tid == 0) s_pivots[t] = s;
    // reciprocal square root of the pivot's residual (hardware rsq, within an ulp or so)
    const float rs = __builtin_amdgcn_rsqf(gs);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int row = ra + p;
      const float gi = __builtin_amdgcn_exp2f(hk[p] * bl2e) - corr[p];
      const float f = row < n ? gi * rs : 0.f;
      fr[p][t] = f;
      dg[p] = (row == s) ? 0.f : dg[p] - f * f;
    }
    if (va) {
      sF[ra * FS + t] = fr[0][t];
      if (vb) {
        sF[(ra + 1) * FS + t] = fr[1][t];
        reinterpret_cast<float2*>(sDg + (buf ^ 1) * DGS)[tid] = make_float2(dg[0], dg[1]);
      } else {
        sDg[(buf ^ 1) * DGS + ra] = dg[0];
      }
    }
    __syncthreads();
  });
  __syncthreads();  // a breakdown step leaves the loop before its barrier
  // the thread's two value rows, requested now (the key registers are free) so that their
  // latency overlaps the hand-over; zero past the last key
  uint4 vra[DV / 8], vrb[DV / 8];
  if (a.O) {
    const uint4* srca = reinterpret_cast<const uint4*>(a.V + ((size_t)h * n + ra) * DV);
    const uint4* srcb = reinterpret_cast<const uint4*>(a.V + ((size_t)h * n + ra + 1) * DV);
#pragma unroll
    for (int q = 0; q < DV / 8; ++q) {
      vra[q] = va ? srca[q] : uint4{0u, 0u, 0u, 0u};
      vrb[q] = vb ? srcb[q] : uint4{0u, 0u, 0u, 0u};
    }
  }

  // the trace after the last step when all r steps completed, zero past a breakdown step (the
  // steps taken stored theirs in the loop); pivots, -1 past the rank
  if (a.trace) {
    double Tr = 0.0;
    if (rk == r) {
      const float2 d0p = reinterpret_cast<const float2*>(sDg + (r & 1) * DGS)[lane];
      const float2 d1p = reinterpret_cast<const float2*>(sDg + (r & 1) * DGS)[64 + lane];
      PairScan q0, q1;
      pair_scan2(d0p, d1p, q0, q1);
      Tr = readlane_d(q0.x, 63) + readlane_d(q1.x, 63);
    }
    if (tid <= r && (tid > rk || tid == r)) a.trace[(size_t)h * (r + 1) + tid] = tid < r ? 0.0 : Tr;
  }
  if (a.pivots && tid < r) a.pivots[(size_t)h * r + tid] = tid < rk ? s_pivots[tid] : -1;
  if (tid == 0) {
    a.rank[h] = rk;
    a.flags[h] = flg;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = ra + p;
    if (row >= n) continue;
    if (a.F) {
#pragma unroll
      for (int j = 0; j < R; ++j)
        if (j < r) a.F[((size_t)h * r + j) * n + row] = fr[p][j];
    }
    if (a.diag) a.diag[(size_t)h * n + row] = dg[p];
  }
  if (!a.O) return;  // pivot loop only

  // ---------------- hand over to the weights and attention buffers ----------------
  // L = F[S, :] (lower triangle) and the coreset keys K_S are read out of the loop region
  // into registers; after the barrier the phase-2 buffers reuse those bytes.
  float lrow[R];
  if (tid < R) {
    const int sp = tid < rk ? s_pivots[tid] : 0;
#pragma unroll
    for (int j = 0; j < R; ++j) lrow[j] = (tid < rk && j <= tid) ? sF[sp * FS + j] : 0.f;
  }
  constexpr int KSE = R * (D / 8);                     // uint4 of K_S
  constexpr int KSV = (KSE + NT - 1) / NT;             // per thread
  uint4 ksv[KSV];
#pragma unroll
  for (int i = 0; i < KSV; ++i) {
    const int e = tid + NT * i, j = e / (D / 8), q = e % (D / 8);
    ksv[i] = (e < KSE && j < rk) ? reinterpret_cast<const uint4*>(sK + s_pivots[j] * D2)[q]
                                 : uint4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  unsigned char* s_A = s_dyn;
  __bf16* s_Ks = reinterpret_cast<__bf16*>(s_dyn + S::KS_OFF);
  __bf16* s_Wp = reinterpret_cast<__bf16*>(s_dyn + S::WP_OFF);
  float* s_Wden = reinterpret_cast<float*>(s_dyn + S::WDEN_OFF);
  float (*s_L)[S::LS] = reinterpret_cast<float (*)[S::LS]>(s_dyn + S::L_OFF);
  if (tid < R) {
#pragma unroll
    for (int j = 0; j < R; ++j) s_L[tid][j] = lrow[j];
    s_L[tid][R] = tid < rk ? 1.0f / lrow[tid] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < KSV; ++i) {
    const int e = tid + NT * i, j = e / (D / 8), q = e % (D / 8);
    if (e < KSE) *reinterpret_cast<uint4*>(s_Ks + j * S::KSP + 8 * q) = ksv[i];
  }

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
  for (int c0 = 0; c0 < 2 * NT; c0 += CH) {
    __syncthreads();
    if (ra >= c0 && ra < c0 + CH) {
      // the thread's two rows are adjacent columns of F^T and V^T: one 32-bit store per pair
      const int ii = ra - c0;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        __bf16 ha, la, hb, lb;
        split_bf16(fr[0][j], ha, la);
        split_bf16(fr[1][j], hb, lb);
        *reinterpret_cast<uint32_t*>(FtH + j * CH + ii) =
            (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
        *reinterpret_cast<uint32_t*>(FtL + j * CH + ii) =
            (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
      }
#pragma unroll
      for (int q = 0; q < DV / 8; ++q) {
        const uint32_t wa[4] = {vra[q].x, vra[q].y, vra[q].z, vra[q].w};
        const uint32_t wb[4] = {vrb[q].x, vrb[q].y, vrb[q].z, vrb[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *reinterpret_cast<uint32_t*>(Vt + (8 * q + 2 * e) * CH + ii) = (wa[e] & 0xffffu) | (wb[e] << 16);
          *reinterpret_cast<uint32_t*>(Vt + (8 * q + 2 * e + 1) * CH + ii) = (wa[e] >> 16) | (wb[e] & 0xffff0000u);
        }
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
  // backward substitution L^T W = X, one column per thread, W in place of X.  Rows at and past
  // the rank need no test: their L rows, reciprocal diagonals and X rows are all zero, so
  // they solve to zero and subtract nothing.
  for (int c = tid; c <= DV; c += NT) {
    float xv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) xv[j] = Xs[j * S::XP + c];
#pragma unroll
    for (int t = R - 1; t >= 0; --t) {
      xv[t] *= s_L[t][R];
#pragma unroll
      for (int j = 0; j < t; ++j) xv[j] = fmaf(-s_L[t][j], xv[t], xv[j]);
    }
    if (a.W) {
      float* Wc = a.W + (size_t)h * r * (DV + 1) + c;
#pragma unroll
      for (int t = 0; t < R; ++t)
        if (t < r) Wc[(size_t)t * (DV + 1)] = xv[t];
    }
    if (c < DV) {
#pragma unroll
      for (int t = 0; t < R; ++t) s_Wp[c * S::WPP + perm32(t)] = (__bf16)xv[t];
    } else {
#pragma unroll
      for (int t = 0; t < R; ++t) s_Wden[t] = xv[t];
    }
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
  using S = ResidentSmem<WC_RES_D, WC_RES_DV, kResidentR, kResidentThreads>;
  const int bytes = S::bytes(a.n);
  if (bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&resident_kernel<WC_RES_D, WC_RES_DV, kResidentR, kResidentThreads>),
        hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((resident_kernel<WC_RES_D, WC_RES_DV, kResidentR, kResidentThreads>), dim3(heads),
                     dim3(kResidentThreads), bytes, st, a);
  return hipGetLastError();
}

}  // namespace wc
