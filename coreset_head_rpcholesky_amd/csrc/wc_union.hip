// Nystroem weights over the union of the bins' coresets (divide-and-conquer WildCat,
// gist.science/de/paper/2602.10056, "Methodik" part 1 efficiency: B bins chosen in parallel;
// part 2: once K_S is chosen, W = h(K_S, K_S)^+ h(K_S, K), with the all-ones column appended
// for the softmax normaliser):
//     H_SS W = X,   X = exp(beta K_S K^T) [V, 1]   (X comes from the attention kernels).
//
// The pseudo-inverse is taken by a Cholesky of H_SS in slot order that leaves out every point
// whose residual is at most tol H_jj (numerically in the span of the earlier points; for
// distinct keys nothing is left out and this is the inverse).  A left-out point j is a zero
// column of L; with L~ the factor whose left-out rows and columns are replaced by unit ones,
// M = L~^{-1} with the left-out rows zeroed is the inverse of the kept part embedded in zeros,
// so W = M^T ... M X keeps the weight rows of left-out points (and of empty slots) at zero.
//
// Blocked right-looking algorithm on 64 x 64 blocks of A = H_SS (fp32), per block column k:
//   diag    one workgroup per head eliminates A_kk with the drop rule and forms M_kk (block 0
//           in a launch of its own, block k+1 inside the update of step k);
//   panel   L_ik = A_ik M_kk^T (i > k, in place over A_ik) and Z_k = M_kk X_k (in place);
//   update  A_ij -= L_ik L_jk^T (k < j <= i) and X_i -= L_ik Z_k;
// then the backward substitution, block k from the last: W_k = M_kk^T Z_k and
// Z_j -= L_kj^T W_k for j < k.  All heads run in each launch.
#include "wc_device.h"
#include "wc_elim.h"
#include "wc_kernels.h"

namespace wc {

namespace {

constexpr int kUB = 64;   // block size
constexpr int kLP = 68;   // LDS row pitch (floats) of the staged 64 x 64 operands

__device__ __forceinline__ bool slot_valid(const UnionArgs& a, int h, int j) {
  return j < a.r && a.pivots[(size_t)h * a.r + j] >= 0;
}

// One 64 x 64 x 64 product on a 256-thread workgroup,
//     acc[i][c] += sum_t sP[t][4 ti + i] sQ[t][4 tc + c],  (ti, tc) = (tid / 16, tid % 16),
// with both operands staged k-major in LDS.  Wave w computes the 32 x 32 quarter (w / 2, w % 2)
// on the fp32 matrix cores (32 x 32 x 2 steps over t), then the product passes through sP
// (row-major) so that every thread picks up its 4 x 4 piece; sP is overwritten.  Every thread
// of the workgroup must call it.
__device__ __forceinline__ void mm64(float (*sP)[kLP], const float (*sQ)[kLP], float acc[4][4]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, kh = lane >> 5, m0 = 32 * (w >> 1), n0 = 32 * (w & 1);
  f32x16 c;
#pragma unroll
  for (int v = 0; v < 16; ++v) c[v] = 0.f;
#pragma unroll 8
  for (int t = 0; t < kUB; t += 2)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(sP[t + kh][m0 + l32], sQ[t + kh][n0 + l32], c, 0, 0, 0);
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 16; ++v) sP[m0 + 8 * (v >> 2) + 4 * kh + (v & 3)][n0 + l32] = c[v];
  __syncthreads();
  const int i0 = 4 * (tid >> 4), c0 = 4 * (tid & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q = *reinterpret_cast<const float4*>(&sP[i0 + i][c0]);
    acc[i][0] += q.x; acc[i][1] += q.y; acc[i][2] += q.z; acc[i][3] += q.w;
  }
}

// sT[t][i] = G[i * ld + t] for a 64 x 64 block of a row-major matrix with ld % 4 == 0.
__device__ __forceinline__ void stage_transposed(float (*sT)[kLP], const float* G, size_t ld) {
  const int tid = threadIdx.x, i = tid >> 2, t0 = 16 * (tid & 3);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(G + (size_t)i * ld + t0 + 4 * q);
    sT[t0 + 4 * q + 0][i] = v.x;
    sT[t0 + 4 * q + 1][i] = v.y;
    sT[t0 + 4 * q + 2][i] = v.z;
    sT[t0 + 4 * q + 3][i] = v.w;
  }
}

// sN[t][c] = G[t * ld + c] for a 64 x 64 block of a row-major matrix with ld % 4 == 0.
__device__ __forceinline__ void stage_direct(float (*sN)[kLP], const float* G, size_t ld) {
  const int tid = threadIdx.x, t = tid >> 2, c0 = 16 * (tid & 3);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<float4*>(&sN[t][c0 + 4 * q]) =
        *reinterpret_cast<const float4*>(G + (size_t)t * ld + c0 + 4 * q);
}

// sN[t][c] = X[t][col0 + c] over the columns col0 .. col0 + 63 of an X block (ld = dv + 1,
// not a multiple of 4); columns past ncol are zero.
__device__ __forceinline__ void stage_x(float (*sN)[kLP], const float* X, int ld, int col0, int ncol) {
  for (int e = threadIdx.x; e < kUB * kUB; e += 256) {
    const int t = e >> 6, c = e & 63;
    sN[t][c] = col0 + c < ncol ? X[(size_t)t * ld + col0 + c] : 0.f;
  }
}

__device__ __forceinline__ void zero_acc(float acc[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = 0.f;
}

// ---- gather: the coreset keys as rows, zero rows for empty slots ---------------------------
template <typename T, int D>
__global__ void __launch_bounds__(64) union_gather_kernel(UnionArgs a) {
  const int j = blockIdx.x, h = blockIdx.y;
  const int s = a.pivots[(size_t)h * a.r + j];
  const T* K = reinterpret_cast<const T*>(a.K) + ((size_t)h * a.n + (s >= 0 ? s : 0)) * D;
  T* Qs = reinterpret_cast<T*>(a.Qs) + ((size_t)h * a.r + j) * D;
  for (int e = threadIdx.x; e < D; e += 64) Qs[e] = s >= 0 ? K[e] : T(0);
}

// ---- gram: A = exp(beta K_S K_S^T) on the lower blocks, its diagonal, zero X padding -------
template <typename T, int D>
__global__ void __launch_bounds__(256) union_gram_kernel(UnionArgs a) {
  __shared__ __attribute__((aligned(16))) float sI[32][kLP];
  __shared__ __attribute__((aligned(16))) float sJ[32][kLP];
  const int h = blockIdx.y, tid = threadIdx.x;
  int x = blockIdx.x, bi = 0;
  while (x > bi) x -= ++bi;
  const int bj = x;
  const T* Qs = reinterpret_cast<const T*>(a.Qs) + (size_t)h * a.r * D;
  float acc[4][4];
  zero_acc(acc);
  for (int e0 = 0; e0 < D; e0 += 32) {
    __syncthreads();
    for (int q = tid; q < 2 * kUB * 32; q += 256) {
      const int side = q >> 11, row = (q >> 5) & 63, e = q & 31;
      const int slot = (side ? bj : bi) * kUB + row;
      const float v = slot < a.r ? ld_elem<T>(Qs + (size_t)slot * D + e0 + e) : 0.f;
      (side ? sJ : sI)[e][row] = v;
    }
    __syncthreads();
    const int i0 = 4 * (tid >> 4), c0 = 4 * (tid & 15);
#pragma unroll 8
    for (int e = 0; e < 32; ++e) {
      const float4 p = *reinterpret_cast<const float4*>(&sI[e][i0]);
      const float4 q = *reinterpret_cast<const float4*>(&sJ[e][c0]);
      const float pv[4] = {p.x, p.y, p.z, p.w}, qv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = fmaf(pv[i], qv[c], acc[i][c]);
    }
  }
  const int i0 = 4 * (tid >> 4), c0 = 4 * (tid & 15);
  float* A = a.A + (size_t)h * a.rp * a.rp;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int si = bi * kUB + i0 + i;
    const bool vi = slot_valid(a, h, si);
    float out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int sj = bj * kUB + c0 + c;
      out[c] = vi && slot_valid(a, h, sj) ? expf(a.beta * acc[i][c]) : 0.f;
      if (bi == bj && si == sj) a.Hd[(size_t)h * a.rp + si] = out[c];
    }
    *reinterpret_cast<float4*>(A + (size_t)si * a.rp + bj * kUB + c0) = make_float4(out[0], out[1], out[2], out[3]);
  }
  if (blockIdx.x == 0) {
    const int nc = a.dv + 1;
    float* X = a.X + (size_t)h * a.rp * nc;
    for (int e = a.r * nc + tid; e < a.rp * nc; e += 256) X[e] = 0.f;
  }
}

// ---- diag: M_kk = inverse of the Cholesky factor of the kept part of A_kk -------------------
// Wave 0 of the workgroup eliminates the (already updated) block in sA with the leave-out rule
// (elim_block64_wave); left-out points of valid slots set WC_DFLAG_DEPENDENT.  The diagonal
// entries H_jj (the scale of the leave-out test) are staged in LDS first.
__device__ __forceinline__ void diag_block(const UnionArgs& a, int h, int k, float (*sA)[kLP],
                                           float (*sCol)[kUB], float (*sRow)[kUB], float* sHd) {
  if (threadIdx.x < kUB) sHd[threadIdx.x] = a.Hd[(size_t)h * a.rp + (size_t)k * kUB + threadIdx.x];
  const bool dependent = elim_block64_wave<kLP>(&sA[0][0], sHd, a.tol, sCol);
  store_block<kUB, kLP>(&sA[0][0], a.M + ((size_t)h * (a.rp / kUB) + k) * kUB * kUB);
  if (dependent && threadIdx.x == 0) atomicOr(&a.flags[h], WC_DFLAG_DEPENDENT);
}

// The first diagonal block (later ones are factored by the update of the step before).
__global__ void __launch_bounds__(256) union_diag0_kernel(UnionArgs a) {
  __shared__ __attribute__((aligned(16))) float sA[kUB][kLP];
  __shared__ __attribute__((aligned(16))) float sCol[2][kUB];
  __shared__ __attribute__((aligned(16))) float sRow[2][kUB];
  __shared__ float sHd[kUB];
  const int h = blockIdx.x;
  const float* A = a.A + (size_t)h * a.rp * a.rp;
  stage_direct(sA, A, a.rp);
  __syncthreads();
  diag_block(a, h, 0, sA, sCol, sRow, sHd);
}

// ---- panel: L_ik = A_ik M_kk^T (i > k) and Z_k = M_kk X_k ------------------------------------
__global__ void __launch_bounds__(256) union_panel_kernel(UnionArgs a, int k) {
  __shared__ __attribute__((aligned(16))) float sP[kUB][kLP];
  __shared__ __attribute__((aligned(16))) float sQ[kUB][kLP];
  const int h = blockIdx.y, tid = threadIdx.x, nb = a.rp / kUB, T = nb - k - 1;
  const int nc = a.dv + 1;
  const float* M = a.M + ((size_t)h * nb + k) * kUB * kUB;
  float* A = a.A + (size_t)h * a.rp * a.rp;
  float* X = a.X + (size_t)h * a.rp * nc;
  float acc[4][4];
  zero_acc(acc);
  const int i0 = 4 * (tid >> 4), c0 = 4 * (tid & 15);
  if ((int)blockIdx.x < T) {
    const int i = k + 1 + blockIdx.x;
    float* Aik = A + (size_t)i * kUB * a.rp + (size_t)k * kUB;
    stage_transposed(sP, Aik, a.rp);   // sP[t][row] = A_ik[row][t]
    stage_transposed(sQ, M, kUB);      // sQ[t][c] = M[c][t]
    __syncthreads();
    mm64(sP, sQ, acc);
    __syncthreads();
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<float4*>(Aik + (size_t)(i0 + r4) * a.rp + c0) =
          make_float4(acc[r4][0], acc[r4][1], acc[r4][2], acc[r4][3]);
  } else {
    const int col0 = (blockIdx.x - T) * kUB;
    float* Xk = X + (size_t)k * kUB * nc;
    stage_transposed(sP, M, kUB);      // sP[t][row] = M[row][t]
    stage_x(sQ, Xk, nc, col0, nc);
    __syncthreads();
    mm64(sP, sQ, acc);
    __syncthreads();
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (col0 + c0 + c < nc) Xk[(size_t)(i0 + r4) * nc + col0 + c0 + c] = acc[r4][c];
  }
}

// ---- update: A_ij -= L_ik L_jk^T (k < j <= i), X_i -= L_ik Z_k --------------------------------
// The block (k+1, k+1) has no other writer in this step, so its workgroup also factors it
// (diag_block for block column k+1) once updated.
__global__ void __launch_bounds__(256) union_update_kernel(UnionArgs a, int k) {
  __shared__ __attribute__((aligned(16))) float sP[kUB][kLP];
  __shared__ __attribute__((aligned(16))) float sQ[kUB][kLP];
  __shared__ __attribute__((aligned(16))) float sCol[2][kUB];
  __shared__ __attribute__((aligned(16))) float sRow[2][kUB];
  __shared__ float sHd[kUB];
  const int h = blockIdx.y, tid = threadIdx.x, nb = a.rp / kUB, T = nb - k - 1;
  const int nc = a.dv + 1;
  float* A = a.A + (size_t)h * a.rp * a.rp;
  float* X = a.X + (size_t)h * a.rp * nc;
  const int npairs = T * (T + 1) / 2;
  float acc[4][4];
  zero_acc(acc);
  const int i0 = 4 * (tid >> 4), c0 = 4 * (tid & 15);
  if ((int)blockIdx.x < npairs) {
    int x = blockIdx.x, ii = 0;
    while (x > ii) x -= ++ii;
    const int i = k + 1 + ii, j = k + 1 + x;
    const float* Lik = A + (size_t)i * kUB * a.rp + (size_t)k * kUB;
    const float* Ljk = A + (size_t)j * kUB * a.rp + (size_t)k * kUB;
    stage_transposed(sP, Lik, a.rp);   // sP[t][row] = L_ik[row][t]
    stage_transposed(sQ, Ljk, a.rp);   // sQ[t][c] = L_jk[c][t]
    __syncthreads();
    mm64(sP, sQ, acc);
    float* Aij = A + (size_t)i * kUB * a.rp + (size_t)j * kUB;
    if (i == k + 1) {
      // i == j == k + 1: the next diagonal block, factored here from LDS
      __syncthreads();
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 o = *reinterpret_cast<const float4*>(Aij + (size_t)(i0 + r4) * a.rp + c0);
        *reinterpret_cast<float4*>(&sP[i0 + r4][c0]) =
            make_float4(o.x - acc[r4][0], o.y - acc[r4][1], o.z - acc[r4][2], o.w - acc[r4][3]);
      }
      __syncthreads();
      diag_block(a, h, k + 1, sP, sCol, sRow, sHd);
      return;
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4* p = reinterpret_cast<float4*>(Aij + (size_t)(i0 + r4) * a.rp + c0);
      float4 o = *p;
      o.x -= acc[r4][0]; o.y -= acc[r4][1]; o.z -= acc[r4][2]; o.w -= acc[r4][3];
      *p = o;
    }
  } else {
    const int nxz = (nc + kUB - 1) / kUB;
    const int x = blockIdx.x - npairs, i = k + 1 + x / nxz, col0 = (x % nxz) * kUB;
    const float* Lik = A + (size_t)i * kUB * a.rp + (size_t)k * kUB;
    stage_transposed(sP, Lik, a.rp);
    stage_x(sQ, X + (size_t)k * kUB * nc, nc, col0, nc);
    __syncthreads();
    mm64(sP, sQ, acc);
    float* Xi = X + (size_t)i * kUB * nc;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (col0 + c0 + c < nc) Xi[(size_t)(i0 + r4) * nc + col0 + c0 + c] -= acc[r4][c];
  }
}

// ---- backward substitution step k: W_k = M_kk^T Z_k; Z_j -= L_kj^T W_k (j < k) ---------------
__global__ void __launch_bounds__(256) union_back_kernel(UnionArgs a, int k) {
  __shared__ __attribute__((aligned(16))) float sP[kUB][kLP];
  __shared__ __attribute__((aligned(16))) float sQ[kUB][kLP];
  const int h = blockIdx.y, tid = threadIdx.x, nb = a.rp / kUB;
  const int nc = a.dv + 1, nxz = (nc + kUB - 1) / kUB;
  const int j = blockIdx.x / nxz, col0 = (blockIdx.x % nxz) * kUB;
  const float* M = a.M + ((size_t)h * nb + k) * kUB * kUB;
  const float* A = a.A + (size_t)h * a.rp * a.rp;
  float* X = a.X + (size_t)h * a.rp * nc;
  float acc[4][4];
  zero_acc(acc);
  const int i0 = 4 * (tid >> 4), c0 = 4 * (tid & 15);
  stage_direct(sP, M, kUB);   // sP[t][row] = M[t][row] = (M^T)[row][t]
  stage_x(sQ, X + (size_t)k * kUB * nc, nc, col0, nc);
  __syncthreads();
  mm64(sP, sQ, acc);          // acc = rows of W_k, columns col0 + c
  if (j == k) {
    float* W = a.W + (size_t)h * a.r * nc;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int wr = k * kUB + i0 + r4;
      if (wr >= a.r) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (col0 + c0 + c < nc) W[(size_t)wr * nc + col0 + c0 + c] = acc[r4][c];
    }
    return;
  }
  __syncthreads();
  // sQ <- W_k block, sP[t][row] = L_kj[t][row] (so that the product is L_kj^T W_k)
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
    for (int c = 0; c < 4; ++c) sQ[i0 + r4][c0 + c] = acc[r4][c];
  stage_direct(sP, A + (size_t)k * kUB * a.rp + (size_t)j * kUB, a.rp);
  __syncthreads();
  zero_acc(acc);
  mm64(sP, sQ, acc);
  float* Xj = X + (size_t)j * kUB * nc;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (col0 + c0 + c < nc) Xj[(size_t)(i0 + r4) * nc + col0 + c0 + c] -= acc[r4][c];
}

template <typename T, int D>
hipError_t run_gather(const UnionArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((union_gather_kernel<T, D>), dim3(a.r, a.H), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_gram(const UnionArgs& a, hipStream_t st) {
  const int nb = a.rp / kUB;
  hipLaunchKernelGGL((union_gram_kernel<T, D>), dim3(nb * (nb + 1) / 2, a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_union_gather(const UnionArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 64 ? run_gather<uint16_t, 64>(a, st) : run_gather<uint16_t, 128>(a, st);
  return a.d == 64 ? run_gather<float, 64>(a, st) : run_gather<float, 128>(a, st);
}

hipError_t launch_union_solve(const UnionArgs& a, hipStream_t st) {
  hipError_t e = a.bf16 ? (a.d == 64 ? run_gram<uint16_t, 64>(a, st) : run_gram<uint16_t, 128>(a, st))
                        : (a.d == 64 ? run_gram<float, 64>(a, st) : run_gram<float, 128>(a, st));
  if (e != hipSuccess) return e;
  const int nb = a.rp / kUB, nxz = (a.dv + 1 + kUB - 1) / kUB;
  hipLaunchKernelGGL(union_diag0_kernel, dim3(a.H), dim3(256), 0, st, a);
  for (int k = 0; k < nb; ++k) {
    const int T = nb - k - 1;
    hipLaunchKernelGGL(union_panel_kernel, dim3(T + nxz, a.H), dim3(256), 0, st, a, k);
    if (T > 0)
      hipLaunchKernelGGL(union_update_kernel, dim3(T * (T + 1) / 2 + T * nxz, a.H), dim3(256), 0, st, a, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return launch_union_back(a, st);
}

hipError_t launch_union_back(const UnionArgs& a, hipStream_t st) {
  const int nb = a.rp / kUB, nxz = (a.dv + 1 + kUB - 1) / kUB;
  for (int k = nb - 1; k >= 0; --k) {
    hipLaunchKernelGGL(union_back_kernel, dim3((k + 1) * nxz, a.H), dim3(256), 0, st, a, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wc
