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

// The same elimination of a 64 x 64 block by one wave, without barriers (same results up to
// rounding order).  Called by every thread of the workgroup; wave 0 works and the others wait at
// the final barrier.  Lane i holds row i of the block and column i of G.  Step j reads column j
// of the block (every lane's A[i][j], written to LDS at the end of step j-1) and takes the
// pivot p = A[j][j] and the leave-out scale hd[j] by readlane; rows i > j subtract
// f_i = A[i][j] / p times row j, whose entries past j equal column j's (the block is
// symmetric); column c of G subtracts f_i G[j][c] from its rows i > j.  Row j of
// M = G[j][:] rsq(p) (G's row j is final once step j begins) goes into row j of sA, which was
// read into registers at the start.  One wave's LDS accesses complete in order, so no barrier
// separates a column's write from its reads; the two column buffers alternate.  Returns, in
// thread 0, whether a point with hd > 0 was left out.
template <int P>
__device__ __forceinline__ bool elim_block64_wave(float* sA, const float* hd, float tol, float (*sCol)[64]) {
  constexpr int B = 64;
  bool dependent = false;
  __syncthreads();  // the block and hd are complete in LDS
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const float hdl = hd[lane];  // leave-out scale of the lane's point, broadcast by readlane
    float v[B], g[B];
#pragma unroll
    for (int e = 0; e < B; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(sA + lane * P + e);
      v[e] = x.x; v[e + 1] = x.y; v[e + 2] = x.z; v[e + 3] = x.w;
    }
#pragma unroll
    for (int e = 0; e < B; ++e) g[e] = e == lane ? 1.f : 0.f;
    sCol[0][lane] = v[0];
    static_for<0, B>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const float* col = sCol[j & 1];
      const float p = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), j));
      const float hj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hdl), j));
      const bool keep = p > tol * hj;
      dependent |= !keep && hj > 0.f;
      sA[j * P + lane] = g[j] * (keep ? __builtin_amdgcn_rsqf(p) : 0.f);
      if (keep) {
        const float rp = __builtin_amdgcn_rcpf(p);
        const float f = v[j] * rp, t = g[j] * rp;
        constexpr int k0 = (j + 1) & ~3;
#pragma unroll
        for (int k4 = k0; k4 < B; k4 += 4) {
          const float4 c4 = *reinterpret_cast<const float4*>(col + k4);
          const float c[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (k4 + e > j) {
              v[k4 + e] = fmaf(-f, c[e], v[k4 + e]);
              g[k4 + e] = fmaf(-c[e], t, g[k4 + e]);
            }
          }
        }
      }
      if constexpr (j + 1 < B) sCol[(j + 1) & 1][lane] = v[j + 1];
    });
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
