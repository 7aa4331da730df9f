// Nystroem weights W = H_SS^{-1} H_{S,:} [V, 1] (gist.science/de/paper/2602.10056,
// "Methodik" part 2: W = h(K_S, K_S)^+ h(K_S, K), compressed values V_S = W V; the extra
// column of ones carries the softmax normaliser).
//
// Computed through the partial Cholesky factor F of the pivot loop: with L = F[S, :]
// (lower triangular, L L^T = H_SS) and H_{:,S} = F L^T,
//     W = L^{-T} L^{-1} L F^T [V, 1] = L^{-T} X,   X = F^T [V, 1].
// This skips recomputing exp(beta K_S K^T) and factorising H_SS, and in fp32 it is the more
// accurate of the two orders (L is the factor the pivot loop already formed).
//   1. gather_L:   L[t][j] = F[j][s_t] for j <= t < rank, zero elsewhere.
//   2. x_partial:  X over a chunk of rows on the bf16 matrix cores: F enters as hi + lo bf16
//                  parts (about 16 significant bits), V exactly (bf16 inputs) or as hi + lo
//                  (fp32 inputs); the ones column is an fp32 sum.  Chunks are reduced in a
//                  fixed order (x_reduce), so W is bitwise reproducible.
//   3. trisolve:   blocked backward substitution L^T W = X, 64-row diagonal blocks solved in
//                  registers, the rows above updated with the solved block.
#include "wc_device.h"
#include "wc_kernels.h"

namespace wc {

__global__ void __launch_bounds__(256) gather_L_kernel(WeightsArgs a) {
  const int t = blockIdx.x, h = blockIdx.y;
  const int r = a.r, rk = a.rank[h];
  const int s = (t < rk) ? a.pivots[(size_t)h * r + t] : 0;
  const float* F = a.F + (size_t)h * r * a.n;
  float* L = a.L + ((size_t)h * r + t) * r;
  for (int j = threadIdx.x; j < r; j += 256)
    L[j] = (t < rk && j <= t) ? F[(size_t)j * a.n + s] : 0.f;
}

// X partial over rows [i0, i0 + chunk_rows) for 128 rows of X (j0 .. j0 + 127).
// 4 waves; MFMA tiles (jt < 4) x (ct < DV/32), tile k of wave w is w + 4k.  Each 64-row
// sub-pass of F (hi/lo bf16) and V^T is staged in LDS; the next sub-pass is loaded into
// registers while the matrix cores work on the current one.
constexpr int XJG = 128;  // rows of X per workgroup
constexpr int XSUB = 64;  // key rows per sub-pass

template <typename TV, int DV, bool VEC>
__global__ void __launch_bounds__(256) x_partial_kernel(WeightsArgs a) {
  constexpr int SP = XSUB + 8;          // padded LDS row (bf16)
  constexpr bool SPLITV = sizeof(TV) == 4;
  constexpr int NCT = DV / 32, NTILE = 4 * NCT, TPW = NTILE / 4;
  constexpr int VPT = DV / 4;           // V elements per thread per sub-pass (row ii, quarter cq)
  __shared__ __attribute__((aligned(16))) __bf16 sFh[XJG * SP];
  __shared__ __attribute__((aligned(16))) __bf16 sFl[XJG * SP];
  __shared__ __attribute__((aligned(16))) __bf16 sVh[DV * SP];
  __shared__ __attribute__((aligned(16))) __bf16 sVl[SPLITV ? DV * SP : 8];
  const int jg = blockIdx.x, chunk = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int n = a.n, r = a.r;
  const int j0 = jg * XJG;
  const int i0 = chunk * a.chunk_rows;
  const int i1 = min(n, i0 + a.chunk_rows);
  const float* F = a.F + (size_t)h * r * n;
  const TV* V = reinterpret_cast<const TV*>(a.V) + (size_t)h * n * DV;
  f32x16 acc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[k][v] = 0.f;
  // F: thread owns row j0 + fj, keys 32 fq .. 32 fq + 31 of the sub-pass
  const int fj = tid >> 1, fq = tid & 1;
  const bool frow = j0 + fj < r;
  // V: thread owns key row ii of the sub-pass, value columns VPT cq .. VPT cq + VPT - 1
  const int ii = tid >> 2, cq = tid & 3;
  float colsum = 0.f;
  float fr[32];
  float vr[VPT];
  auto load = [&](int ib) {
    const int ibase = ib + 32 * fq;
    const float* src = F + (size_t)(j0 + fj) * n + ibase;
    if (VEC && frow && ibase + 32 <= i1) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 x = reinterpret_cast<const float4*>(src)[q];
        fr[4 * q] = x.x; fr[4 * q + 1] = x.y; fr[4 * q + 2] = x.z; fr[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) fr[e] = (frow && ibase + e < i1) ? src[e] : 0.f;
    }
    const int i = ib + ii;
    const TV* vs = V + (size_t)i * DV + cq * VPT;
    if (i < i1) {
      if constexpr (sizeof(TV) == 2) {
#pragma unroll
        for (int q = 0; q < VPT / 8; ++q) {
          const uint4 x = reinterpret_cast<const uint4*>(vs)[q];
          const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vr[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
            vr[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < VPT / 4; ++q) {
          const float4 x = reinterpret_cast<const float4*>(vs)[q];
          vr[4 * q] = x.x; vr[4 * q + 1] = x.y; vr[4 * q + 2] = x.z; vr[4 * q + 3] = x.w;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < VPT; ++e) vr[e] = 0.f;
    }
  };
  if (i0 < i1) load(i0);
  for (int ib = i0; ib < i1; ib += XSUB) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x8 hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        colsum += fr[8 * q + e];
        __bf16 hi, lo;
        split_bf16(fr[8 * q + e], hi, lo);
        hv[e] = hi;
        lv[e] = lo;
      }
      *reinterpret_cast<bf16x8*>(sFh + fj * SP + 32 * fq + 8 * q) = hv;
      *reinterpret_cast<bf16x8*>(sFl + fj * SP + 32 * fq + 8 * q) = lv;
    }
#pragma unroll
    for (int e = 0; e < VPT; ++e) {
      const int c = cq * VPT + e;
      if (SPLITV) {
        __bf16 hi, lo;
        split_bf16(vr[e], hi, lo);
        sVh[c * SP + ii] = hi;
        sVl[c * SP + ii] = lo;
      } else {
        sVh[c * SP + ii] = (__bf16)vr[e];
      }
    }
    __syncthreads();
    if (ib + XSUB < i1) load(ib + XSUB);  // next sub-pass in flight during the MFMAs
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int tile = wid + 4 * k;
      const int jt = tile / NCT, ct = tile % NCT;
      if (j0 + jt * 32 >= r) continue;
#pragma unroll
      for (int kk = 0; kk < XSUB; kk += 16) {
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(sFh + (jt * 32 + l32) * SP + kk + 8 * g);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(sFl + (jt * 32 + l32) * SP + kk + 8 * g);
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(sVh + (ct * 32 + l32) * SP + kk + 8 * g);
        acc[k] = mfma32(ah, bh, acc[k]);
        acc[k] = mfma32(al, bh, acc[k]);
        if (SPLITV) {
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(sVl + (ct * 32 + l32) * SP + kk + 8 * g);
          acc[k] = mfma32(ah, bl, acc[k]);
        }
      }
    }
  }
  float* X = a.Xpart + (((size_t)h * a.nchunk + chunk) * r) * (DV + 1);
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int tile = wid + 4 * k;
    const int jt = tile / NCT, ct = tile % NCT;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = j0 + jt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (j < r) X[(size_t)j * (DV + 1) + ct * 32 + l32] = acc[k][v];
    }
  }
  colsum += __shfl_xor(colsum, 1, 64);
  if (fq == 0 && frow) X[(size_t)(j0 + fj) * (DV + 1) + DV] = colsum;
}

__global__ void __launch_bounds__(256) x_reduce_kernel(WeightsArgs a) {
  const size_t per = (size_t)a.r * (a.dv + 1);
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y;
  if (e >= per) return;
  const float* P = a.Xpart + (size_t)h * a.nchunk * per + e;
  float s = 0.f;
  for (int c = 0; c < a.nchunk; ++c) s += P[(size_t)c * per];
  a.X[(size_t)h * per + e] = s;
}

// Backward substitution L^T W = X for 32 columns of one head.
__global__ void __launch_bounds__(256) trisolve_kernel(WeightsArgs a) {
  constexpr int B = 64;
  __shared__ float sLbb[B][B + 1];
  __shared__ float sW[B][33];
  __shared__ float sLt[B][33];
  const int cg = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = a.r, nc = a.dv + 1, rk = a.rank[h];
  const int c0 = cg * 32;
  const float* L = a.L + (size_t)h * r * r;
  float* X = a.X + (size_t)h * r * nc;
  float* W = a.W + (size_t)h * r * nc;
  const int nb = (rk + B - 1) / B;
  for (int bi = nb - 1; bi >= 0; --bi) {
    const int b0 = bi * B, bs = min(B, rk - b0);
    __syncthreads();
    for (int e = tid; e < B * B; e += 256) {
      const int i = e / B, j = e % B;
      sLbb[i][j] = (i < bs && j < bs) ? L[(size_t)(b0 + i) * r + b0 + j] : 0.f;
    }
    for (int e = tid; e < B * 32; e += 256) {
      const int i = e / 32, c = e % 32;
      sW[i][c] = (i < bs && c0 + c < nc) ? X[(size_t)(b0 + i) * nc + c0 + c] : 0.f;
    }
    __syncthreads();
    if (tid < 32) {
      float xv[B];
#pragma unroll
      for (int i = 0; i < B; ++i) xv[i] = sW[i][tid];
#pragma unroll
      for (int tt = B - 1; tt >= 0; --tt) {
        if (tt < bs) {
          const float w = xv[tt] / sLbb[tt][tt];
          xv[tt] = w;
#pragma unroll
          for (int j = 0; j < tt; ++j) xv[j] = fmaf(-sLbb[tt][j], w, xv[j]);
        }
      }
#pragma unroll
      for (int i = 0; i < B; ++i) sW[i][tid] = xv[i];
    }
    __syncthreads();
    for (int e = tid; e < B * 32; e += 256) {
      const int i = e / 32, c = e % 32;
      if (i < bs && c0 + c < nc) W[(size_t)(b0 + i) * nc + c0 + c] = sW[i][c];
    }
    // X[j][c] -= sum_tt L[b0 + tt][j] W[b0 + tt][c] for the rows j < b0 above the block
    for (int jb = 0; jb < b0; jb += 32) {
      __syncthreads();
      for (int e = tid; e < B * 32; e += 256) {
        const int tt = e / 32, jj = e % 32;
        sLt[tt][jj] = (tt < bs) ? L[(size_t)(b0 + tt) * r + jb + jj] : 0.f;
      }
      __syncthreads();
      const int c = tid & 31;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int jj = (tid >> 5) + 8 * k;
        float acc = 0.f;
#pragma unroll 8
        for (int tt = 0; tt < B; ++tt) acc = fmaf(sLt[tt][jj], sW[tt][c], acc);
        if (c0 + c < nc) X[(size_t)(jb + jj) * nc + c0 + c] -= acc;
      }
    }
  }
  // rows after the rank are zero
  for (int e = tid; e < (r - rk) * 32; e += 256) {
    const int i = rk + e / 32, c = e % 32;
    if (c0 + c < nc) W[(size_t)i * nc + c0 + c] = 0.f;
  }
}

// Inverses of L's 64 x 64 diagonal blocks (the part before the rank; zero past it), for the
// blocked back substitution.  Grid (r/64, heads), one thread per column of the inverse: forward
// substitution down the column, x_i = (delta_ic - sum_{c <= j < i} L_ij x_j) / L_ii.
__global__ void __launch_bounds__(64) tri_inv_kernel(WeightsArgs a) {
  constexpr int B = 64, P = B + 4;
  __shared__ __attribute__((aligned(16))) float sL[B][P];
  __shared__ float sR[B];
  const int b = blockIdx.x, h = blockIdx.y, c = threadIdx.x, r = a.r;
  const int b0 = b * B, bs = max(0, min(B, a.rank[h] - b0));
  const float* L = a.L + (size_t)h * r * r;
#pragma unroll 4
  for (int i = 0; i < B; ++i) sL[i][c] = (i < bs && c < bs) ? L[(size_t)(b0 + i) * r + b0 + c] : 0.f;
  __syncthreads();
  sR[c] = c < bs ? 1.0f / sL[c][c] : 0.f;
  __syncthreads();
  float x[B];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    float acc0 = i == c ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
    for (int j = 0; j + 1 < i; j += 2) {
      acc0 = fmaf(-sL[i][j], x[j], acc0);
      acc1 = fmaf(-sL[i][j + 1], x[j + 1], acc1);
    }
    if (i & 1) acc0 = fmaf(-sL[i][i - 1], x[i - 1], acc0);
    // x_j = 0 for j < c, so the sum may run over all j < i
    x[i] = (i >= c && i < bs && c < bs) ? (acc0 + acc1) * sR[i] : 0.f;
  }
  float* M = a.Minv + ((size_t)h * (r / B) + b) * B * B;
#pragma unroll
  for (int i = 0; i < B; ++i) M[i * B + c] = x[i];
}

template <typename TV, int DV>
static hipError_t run_weights(const WeightsArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(gather_L_kernel, dim3(a.r, a.H), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 xg((a.r + XJG - 1) / XJG, a.nchunk, a.H);
  if (a.n % 4 == 0 && a.chunk_rows % 4 == 0)
    hipLaunchKernelGGL((x_partial_kernel<TV, DV, true>), xg, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((x_partial_kernel<TV, DV, false>), xg, dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t per = (size_t)a.r * (DV + 1);
  hipLaunchKernelGGL(x_reduce_kernel, dim3((unsigned)((per + 255) / 256), a.H), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.Minv) {
    // blocked: every diagonal block inverted at once, then one launch per block
    hipLaunchKernelGGL(tri_inv_kernel, dim3(a.r / 64, a.H), dim3(64), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    UnionArgs u{};
    u.H = a.H; u.dv = a.dv; u.r = a.r; u.rp = a.r;
    u.A = a.L; u.M = a.Minv; u.X = a.X; u.W = a.W;
    return launch_union_back(u, st);
  }
  hipLaunchKernelGGL(trisolve_kernel, dim3((DV + 1 + 31) / 32, a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_weights(const WeightsArgs& a, hipStream_t st) {
  if (a.bf16) return a.dv == 64 ? run_weights<uint16_t, 64>(a, st) : run_weights<uint16_t, 128>(a, st);
  return a.dv == 64 ? run_weights<float, 64>(a, st) : run_weights<float, 128>(a, st);
}

// Divide-and-conquer selection ran bin b of head h as sub-head h B + b; its pivots become key
// indices of the head (offset b n/B) in slots b r/B .., empty slots keep -1, and the ranks
// and flags of the bins are folded per head.
__global__ void __launch_bounds__(256) bins_combine_kernel(BinsArgs a) {
  const int h = blockIdx.x, r = a.B * a.rb;
  int taken = 0;
  uint32_t fl = 0u;
  for (int j = threadIdx.x; j < r; j += 256) {
    const int b = j / a.rb, sub = h * a.B + b;
    const int s = a.piv_sub[(size_t)sub * a.rb + j % a.rb];
    a.pivots[(size_t)h * r + j] = s >= 0 ? s + b * a.nb : -1;
  }
  if (threadIdx.x == 0) {
    for (int b = 0; b < a.B; ++b) {
      taken += a.rank_sub[h * a.B + b];
      fl |= a.flags_sub[h * a.B + b];
    }
    a.rank[h] = taken;
    a.flags[h] = fl;
    a.rank_slots[h] = r;
  }
}

hipError_t launch_bins_combine(const BinsArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bins_combine_kernel, dim3(a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace wc
