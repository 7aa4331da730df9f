// Elimination of a small symmetric block with the leave-out rule, shared by the union weights
// and the block pivot selection.
#pragma once
#include "wc_device.h"

namespace wc {

// M = inverse of the Cholesky factor of the kept part of the B x B block in sA (row-major,
// pitch P floats), for a workgroup of 4 B threads; M replaces the block in sA (same pitch).  Right-looking elimination applied
// alongside to the identity: step j takes the pivot residual p = A[j][j]; if p > tol hd[j]
// every later row i subtracts f_i = A[i][j] / p times row j, in the block and in G (G starts
// as the identity).  G ends as U^{-1}, U the unit lower factor of A = U diag(p) U^T over the
// kept points, so M = diag(p)^{-1/2} G; a left-out point eliminates nothing and gets a zero
// row of M (M[j][j] > 0 exactly for the kept ones).  Thread (i, q) holds columns
// q B/4 .. (q+1) B/4 - 1 of row i of the block and of G; column j of the block and row j of G
// are published in LDS (double-buffered by the parity of j, one barrier per step).  hd (B
// entries) should sit in LDS: it is read at every step.  Ends with a barrier.  Returns, in
// every thread, whether a point with hd > 0 was left out.
template <int B, int P>
__device__ __forceinline__ bool elim_block(float* sA, const float* hd, float tol,
                                           float (*sCol)[B], float (*sRow)[B]) {
  constexpr int CB = B / 4;
  const int tid = threadIdx.x, ri = tid >> 2, q = tid & 3, c0 = CB * q;
  float v[CB], g[CB];
#pragma unroll
  for (int e = 0; e < CB; e += 4) {
    const float4 x = *reinterpret_cast<const float4*>(sA + ri * P + c0 + e);
    v[e] = x.x; v[e + 1] = x.y; v[e + 2] = x.z; v[e + 3] = x.w;
  }
#pragma unroll
  for (int e = 0; e < CB; ++e) g[e] = ri == c0 + e ? 1.f : 0.f;
  bool dependent = false;
  __syncthreads();  // sA may be overwritten by the caller only after everyone has read it
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int buf = j & 1;
    if (q == j / CB) sCol[buf][ri] = v[j % CB];
    if (ri == j) {
#pragma unroll
      for (int e = 0; e < CB; e += 4)
        *reinterpret_cast<float4*>(&sRow[buf][c0 + e]) = make_float4(g[e], g[e + 1], g[e + 2], g[e + 3]);
    }
    __syncthreads();
    const float p = sCol[buf][j];
    const float hj = hd[j];
    const bool keep = p > tol * hj;
    dependent |= !keep && hj > 0.f;
    if (ri == j) {
      // row j of M, into the block's own LDS rows (read once at the start; a global store
      // here would hold up every later barrier until it completes); hardware reciprocal
      // square root, about 1 ulp
      const float s = keep ? __builtin_amdgcn_rsqf(p) : 0.f;
#pragma unroll
      for (int e = 0; e < CB; e += 4)
        *reinterpret_cast<float4*>(sA + j * P + c0 + e) = make_float4(g[e] * s, g[e + 1] * s, g[e + 2] * s, g[e + 3] * s);
    }
    if (keep && ri > j) {
      const float f = sCol[buf][ri] * __builtin_amdgcn_rcpf(p);
#pragma unroll
      for (int e = 0; e < CB; e += 4) {
        const float4 cj = *reinterpret_cast<const float4*>(&sCol[buf][c0 + e]);
        const float4 gj = *reinterpret_cast<const float4*>(&sRow[buf][c0 + e]);
        v[e] = fmaf(-f, cj.x, v[e]); v[e + 1] = fmaf(-f, cj.y, v[e + 1]);
        v[e + 2] = fmaf(-f, cj.z, v[e + 2]); v[e + 3] = fmaf(-f, cj.w, v[e + 3]);
        g[e] = fmaf(-f, gj.x, g[e]); g[e + 1] = fmaf(-f, gj.y, g[e + 1]);
        g[e + 2] = fmaf(-f, gj.z, g[e + 2]); g[e + 3] = fmaf(-f, gj.w, g[e + 3]);
      }
    }
  }
  __syncthreads();
  return dependent;
}

// The elimination of a 32 x 32 block by one wave, rows and identity image side by side: lanes
// 0-31 hold the rows of the block, lanes 32-63 the columns of G (the image of the identity), so
// one fused multiply-add per entry and pivot updates both (rows i > j subtract f_i times row j,
// column c of G subtracts G[j][c] / p times column j of the block: the same form
// w[k] -= c[k] (w[j] / p) with c column j of the block).  Column j+1 is written to LDS by the
// row lanes as soon as step j has updated it, before the rest of step j, and read back by every
// lane in step j+1 (one wave's LDS accesses complete in order, so no barrier separates them; two
// buffers alternate).  The pivot p and its leave-out scale come by readlane; a left-out pivot
// turns the step's multiplier to zero rather than skipping it, so the step is straight-line
// code.  Row j of M = G[j][:] rsq(p) is written by the G lanes to sM (pitch PM): G's row j is
// final once step j begins.
// The block sits in sA with pitch PA, hd are the 32 leave-out scales.  Wave 0 only; returns,
// in every lane of it, whether a point with hd > 0 was left out.
template <int PA, int PM>
__device__ __forceinline__ bool elim32_wave(const float* sA, const float* hd, float tol, float (*sCol)[64],
                                            float* sM) {
  constexpr int B = 32;
  const int lane = threadIdx.x & 63, i = lane & 31;
  const bool rowlane = lane < 32;
  const float hdl = hd[i];
  float w[B];
#pragma unroll
  for (int e = 0; e < B; e += 4) {
    const float4 x = *reinterpret_cast<const float4*>(sA + i * PA + e);
    w[e] = rowlane ? x.x : (e == i ? 1.f : 0.f);
    w[e + 1] = rowlane ? x.y : (e + 1 == i ? 1.f : 0.f);
    w[e + 2] = rowlane ? x.z : (e + 2 == i ? 1.f : 0.f);
    w[e + 3] = rowlane ? x.w : (e + 3 == i ? 1.f : 0.f);
  }
  if (rowlane) sCol[0][i] = w[0];
  bool dependent = false;
  static_for<0, B>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const float* col = sCol[j & 1];
    const float p = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[j]), j));
    const float hj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hdl), j));
    const bool keep = p > tol * hj;
    dependent |= !keep && hj > 0.f;
    const float rs = keep ? __builtin_amdgcn_rsqf(p) : 0.f;
    const float sc = keep ? w[j] * __builtin_amdgcn_rcpf(p) : 0.f;
    if (!rowlane) sM[j * PM + i] = w[j] * rs;
    if constexpr (j + 1 < B) {
      // the float4 group holding column j+1 first, then its publication, then the rest
      constexpr int g1 = (j + 1) & ~3;
      {
        const float4 c4 = *reinterpret_cast<const float4*>(col + g1);
        const float c[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (g1 + e > j) w[g1 + e] = fmaf(-c[e], sc, w[g1 + e]);
      }
      if (rowlane) sCol[(j + 1) & 1][i] = w[j + 1];
#pragma unroll
      for (int k4 = g1 + 4; k4 < B; k4 += 4) {
        const float4 c4 = *reinterpret_cast<const float4*>(col + k4);
        w[k4] = fmaf(-c4.x, sc, w[k4]);
        w[k4 + 1] = fmaf(-c4.y, sc, w[k4 + 1]);
        w[k4 + 2] = fmaf(-c4.z, sc, w[k4 + 2]);
        w[k4 + 3] = fmaf(-c4.w, sc, w[k4 + 3]);
      }
      // the step's updates happen in this step: otherwise the compiler defers them to each
      // entry's first use and keeps every earlier column and multiplier live in registers
#pragma unroll
      for (int k = j + 1; k < B; ++k) asm volatile("" : "+v"(w[k]));
    }
  });
  return dependent;
}

// 32 x 32 x 32 product on a 256-thread workgroup: wave w forms the 16 x 16 quarter
// (w / 2, w % 2) on the fp32 matrix cores (16 x 16 x 4: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; the result rows are 4 (l / 16) .. + 3 of column l % 16) and hands each
// entry (row, column, value) to out.
template <class FA, class FB, class FO>
__device__ __forceinline__ void mm32_quarters(FA a_at, FB b_at, FO out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lk = lane >> 4, r0 = 16 * (w >> 1), c0 = 16 * (w & 1);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a_at(r0 + lr, 4 * s + lk), b_at(4 * s + lk, c0 + lr), acc, 0, 0, 0);
#pragma unroll
  for (int v = 0; v < 4; ++v) out(r0 + 4 * lk + v, c0 + lr, acc[v]);
}

// M = inverse of the Cholesky factor of the kept part of a 64 x 64 block (elim_block's result,
// up to rounding order), in two halves of 32 pivots, for a 256-thread workgroup.  With
// D = [D11 D21^T; D21 D22]:
//   M11 = elimination of D11 (elim32_wave),  L21 = D21 M11^T,  D22' = D22 - L21 L21^T,
//   M22 = elimination of D22',  M21 = -M22 L21 M11,
// and M = [M11 0; M21 M22] replaces the block in sA (pitch P).  A point left out in the first
// half has a zero row in M11 and so a zero column in L21; one left out in the second half has a
// zero row in M22 and so in M21: M is the inverse of the kept part's factor with zero rows for
// the left-out points, as before.  sS holds 4 x 32 x 33 floats of scratch.  Every thread calls
// it; ends with a barrier; returns, in thread 0, whether a point with hd > 0 was left out.
template <int P>
__device__ __forceinline__ bool elim_block64_split(float* sA, const float* hd, float tol, float* sS,
                                                   float (*sCol)[64]) {
  constexpr int PS = 33;
  float* sM1 = sS;
  float* sL = sS + 32 * PS;
  float* sM2 = sS + 2 * 32 * PS;
  float* sT = sS + 3 * 32 * PS;
  const int tid = threadIdx.x;
  bool dependent = false;
  __syncthreads();  // the block and hd are complete in LDS
  if (tid < 64) dependent = elim32_wave<P, PS>(sA, hd, tol, sCol, sM1);
  __syncthreads();
  // L21 = D21 M11^T
  mm32_quarters([&](int r, int t) { return sA[(32 + r) * P + t]; }, [&](int t, int c) { return sM1[c * PS + t]; },
                [&](int r, int c, float v) { sL[r * PS + c] = v; });
  __syncthreads();
  // D22 -= L21 L21^T
  mm32_quarters([&](int r, int t) { return sL[r * PS + t]; }, [&](int t, int c) { return sL[c * PS + t]; },
                [&](int r, int c, float v) { sA[(32 + r) * P + 32 + c] -= v; });
  __syncthreads();
  if (tid < 64) dependent |= elim32_wave<P, PS>(sA + 32 * P + 32, hd + 32, tol, sCol, sM2);
  __syncthreads();
  // T = L21 M11
  mm32_quarters([&](int r, int t) { return sL[r * PS + t]; }, [&](int t, int c) { return sM1[t * PS + c]; },
                [&](int r, int c, float v) { sT[r * PS + c] = v; });
  __syncthreads();
  // M21 = -M22 T, and M assembled over the block
  mm32_quarters([&](int r, int t) { return sM2[r * PS + t]; }, [&](int t, int c) { return sT[t * PS + c]; },
                [&](int r, int c, float v) { sA[(32 + r) * P + c] = -v; });
  for (int e = tid; e < 32 * 32; e += blockDim.x) {
    const int r = e >> 5, c = e & 31;
    sA[r * P + c] = sM1[r * PS + c];
    sA[r * P + 32 + c] = 0.f;
    sA[(32 + r) * P + 32 + c] = sM2[r * PS + c];
  }
  __syncthreads();
  return dependent;
}

// Copy M (B x B, pitch P in LDS, as elim_block leaves it) to global memory, row-major with
// leading dimension B, by the 4 B threads of the workgroup.
template <int B, int P>
__device__ __forceinline__ void store_block(const float* sM, float* M) {
  for (int e = threadIdx.x; e < B * B / 4; e += 4 * B) {
    const int row = (4 * e) / B, col = (4 * e) % B;
    *reinterpret_cast<float4*>(M + (size_t)row * B + col) = *reinterpret_cast<const float4*>(sM + row * P + col);
  }
}

}  // namespace wc
