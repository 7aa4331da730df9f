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
  const int sp = (t < rk) ? a.pivots[(size_t)h * r + t] : 0;
  const bool valid = t < rk && wc_index_ok(sp, a.n, a.flags ? a.flags + h : nullptr);
  const int s = valid ? sp : 0;
  const float* F = a.F + (size_t)h * r * a.n;
  float* L = a.L + ((size_t)h * r + t) * r;
  for (int j = threadIdx.x; j < r; j += 256)
    L[j] = (valid && j <= t) ? F[(size_t)j * a.n + s] : 0.f;
}

// X partial over the key rows [i0, i0 + chunk_rows) for XJG rows of X.  Eight waves; wave w
// owns the 32 rows j0 + 32 w .. of X and forms them on the bf16 matrix cores,
//   X[j, c] += sum_i F[j, i] V[i, c]   (32 x 32 x 16 MFMAs, one tile per 32 value columns),
// its A operand (8 consecutive keys of one row of F) loaded straight from global memory into
// registers and split there into hi + lo bf16 parts, so each element of F is read once in the
// whole grid.  The B operand, V transposed, is staged in LDS once per 64-key sub-pass for all
// eight waves (double-buffered: the next sub-pass's F and V loads are in flight during the
// current MFMAs).  The ones column X[j, dv] = sum_i F[j, i] is an fp32 sum in registers.
// The loads are branch-free (clamped addresses, out-of-range values zeroed where they are
// used), V's before F's in each sub-pass, and the two F buffers alternate without copies, so
// that no wait for one load holds up the loads behind it: the compiler waits for each F
// fragment just before its products and for V just before it is staged.
// Workgroups that share a chunk of keys (and so its rows of V) are dealt to one XCD, so V is
// read from HBM about once and from that XCD's L2 by the others.
constexpr int XW = 8;           // waves per workgroup
constexpr int XJG = 32 * XW;    // rows of X per workgroup
constexpr int XKS = 64;         // key rows per sub-pass
constexpr int XKK = XKS / 16;   // 16-key MFMA steps per sub-pass
constexpr int XVP = XKS + 8;    // LDS pitch (bf16) of one transposed value column

template <typename TV, int DV, bool VEC>
__global__ void __launch_bounds__(64 * XW) x_partial_kernel(WeightsArgs a) {
  constexpr bool SPLITV = sizeof(TV) == 4;
  constexpr int NCT = DV / 32;
  __shared__ __attribute__((aligned(16))) __bf16 sVh[2][DV * XVP];
  __shared__ __attribute__((aligned(16))) __bf16 sVl[SPLITV ? 2 : 1][SPLITV ? DV * XVP : 8];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int n = a.n, r = a.r;
  // workgroup -> (row group, key chunk, head); the row groups of one chunk are consecutive
  // among the workgroups of one XCD (workgroups are dealt to the XCDs round-robin by id)
  const int JG = (r + XJG - 1) / XJG, total = JG * a.nchunk * a.H, L = blockIdx.x;
  const int p = total % 8 == 0 ? (L % 8) * (total / 8) + L / 8 : L;
  const int jg = p % JG, chunk = (p / JG) % a.nchunk, h = p / JG / a.nchunk;
  const int j0 = jg * XJG;
  const int i0 = chunk * a.chunk_rows;
  const int i1 = min(n, i0 + a.chunk_rows);
  const int j = j0 + 32 * wid + l32;  // this lane's row of X (and of F)
  const bool jv = j < r;
  const float* Fj = a.F + ((size_t)h * r + (jv ? j : 0)) * n;
  const TV* V = reinterpret_cast<const TV*>(a.V) + (size_t)h * n * DV;

  // MFMA step kk takes, in lane half g, the keys key_of(kk) .. + 7 of the sub-pass (A and B alike)
  auto key_of = [&](int kk) { return 16 * kk + 8 * g; };
  // F: keys ib + key_of(kk) .. + 7 of row j, kk = 0 .. XKK - 1
  // (VEC: 16-byte loads with no conditions around them.  i1 is a multiple of 4, so each
  // 4-key piece lies wholly inside or wholly past the chunk; a piece past it reads the row's
  // first keys instead, as rows past r read row 0 of the head, and all are zeroed where they
  // are used)
  auto load_f = [&](int ib, float (&f)[XKK][8]) {
#pragma unroll
    for (int kk = 0; kk < XKK; ++kk) {
      const int i = ib + key_of(kk);
      if constexpr (VEC) {
        const float4 x0 = *reinterpret_cast<const float4*>(Fj + (i < i1 ? i : 0));
        const float4 x1 = *reinterpret_cast<const float4*>(Fj + (i + 4 < i1 ? i + 4 : 0));
        f[kk][0] = x0.x; f[kk][1] = x0.y; f[kk][2] = x0.z; f[kk][3] = x0.w;
        f[kk][4] = x1.x; f[kk][5] = x1.y; f[kk][6] = x1.z; f[kk][7] = x1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[kk][e] = (jv && i + e < i1) ? Fj[i + e] : 0.f;
      }
    }
  };
  // V: thread owns key pair (2 kp, 2 kp + 1) of the sub-pass and 16 bytes of value columns;
  // the two keys of each column are packed into one 32-bit LDS word of the transposed layout
  constexpr int CPL = 16 / (int)sizeof(TV);        // value columns per 16-byte load
  constexpr int CG = DV / CPL;                     // column groups
  constexpr int NUNIT = (XKS / 2) * CG;                       // (key pair, column group) units
  constexpr int VPASS = (NUNIT + 64 * XW - 1) / (64 * XW);    // units per thread
  // (keys past the chunk read its last key, and are zeroed when staged)
  auto load_v = [&](int ib, uint4 (&v)[VPASS][2]) {
#pragma unroll
    for (int u = 0; u < VPASS; ++u) {
      const int unit = min(tid + u * 64 * XW, NUNIT - 1), kp = unit / CG, cg = unit % CG;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        v[u][q] = *reinterpret_cast<const uint4*>(V + (size_t)min(ib + 2 * kp + q, i1 - 1) * DV + cg * CPL);
    }
  };
  auto store_v = [&](int ib, int buf, const uint4 (&v)[VPASS][2]) {
#pragma unroll
    for (int u = 0; u < VPASS; ++u) {
      const int unit = tid + u * 64 * XW, kp = unit / CG, cg = unit % CG;
      if (unit >= NUNIT) continue;
      const bool in0 = ib + 2 * kp < i1, in1 = ib + 2 * kp + 1 < i1;
      const uint32_t w0[4] = {in0 ? v[u][0].x : 0u, in0 ? v[u][0].y : 0u, in0 ? v[u][0].z : 0u, in0 ? v[u][0].w : 0u};
      const uint32_t w1[4] = {in1 ? v[u][1].x : 0u, in1 ? v[u][1].y : 0u, in1 ? v[u][1].z : 0u, in1 ? v[u][1].w : 0u};
      if constexpr (!SPLITV) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // columns 8 cg + 2 e and + 1: (key 2kp, key 2kp+1)
          const int c = cg * CPL + 2 * e;
          *reinterpret_cast<uint32_t*>(&sVh[buf][c * XVP + 2 * kp]) = (w0[e] & 0xffffu) | (w1[e] << 16);
          *reinterpret_cast<uint32_t*>(&sVh[buf][(c + 1) * XVP + 2 * kp]) = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // column 4 cg + e, fp32 split into hi + lo bf16 parts
          const int c = cg * CPL + e;
          __bf16 h0, l0, h1, l1;
          split_bf16(__uint_as_float(w0[e]), h0, l0);
          split_bf16(__uint_as_float(w1[e]), h1, l1);
          const bf16x2 hh = {h0, h1}, ll = {l0, l1};
          *reinterpret_cast<bf16x2*>(&sVh[buf][c * XVP + 2 * kp]) = hh;
          *reinterpret_cast<bf16x2*>(&sVl[buf][c * XVP + 2 * kp]) = ll;
        }
      }
    }
  };

  f32x16 acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x16{};
  float colsum = 0.f;
  // products of one sub-pass; F's keys past the chunk and its rows past r count as zero
  auto products = [&](int ib, int buf, const float (&fc)[XKK][8]) {
    const int lim = jv ? i1 - ib - 8 * g : 0;  // keys 16 kk + e of this lane below lim are in range
#pragma unroll
    for (int kk = 0; kk < XKK; ++kk) {
      bf16x8 ah, al;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = 16 * kk + e < lim ? fc[kk][e] : 0.f;
        colsum += x;
        __bf16 hi, lo;
        split_bf16(x, hi, lo);
        ah[e] = hi;
        al[e] = lo;
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int o = (ct * 32 + l32) * XVP + key_of(kk);
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&sVh[buf][o]);
        acc[ct] = mfma32(ah, bh, acc[ct]);
        acc[ct] = mfma32(al, bh, acc[ct]);
        if constexpr (SPLITV) {
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&sVl[buf][o]);
          acc[ct] = mfma32(ah, bl, acc[ct]);
        }
      }
    }
  };
  float fa[XKK][8], fb[XKK][8];
  uint4 vn[VPASS][2];
  if (i0 < i1) {
    load_v(i0, vn);
    load_f(i0, fa);
    store_v(i0, 0, vn);
  }
  __syncthreads();
  // one sub-pass on the F fragments fc, with the next sub-pass's loaded into fn
  // (the loads and the staging run even after the chunk's last sub-pass, from clamped
  // addresses: with no branch around them the compiler neither sinks the loads to their use
  // nor loses count of those in flight; the fence keeps them ahead of the products)
  auto sub_pass = [&](int ib, int buf, const float (&fc)[XKK][8], float (&fn)[XKK][8]) {
    load_v(ib + XKS, vn);
    load_f(ib + XKS, fn);
    __builtin_amdgcn_sched_barrier(0);
    products(ib, buf, fc);
    store_v(ib + XKS, buf ^ 1, vn);
    __syncthreads();
  };
  // sub-passes in pairs (an odd count ends with one wholly past the chunk, all of it zeroed)
  for (int ib = i0; ib < i1; ib += 2 * XKS) {
    sub_pass(ib, 0, fa, fb);
    sub_pass(ib + XKS, 1, fb, fa);
  }
  float* X = a.Xpart + (((size_t)h * a.nchunk + chunk) * r) * (DV + 1);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int jr = j0 + 32 * wid + 8 * (v >> 2) + 4 * g + (v & 3);
      if (jr < r) X[(size_t)jr * (DV + 1) + ct * 32 + l32] = acc[ct][v];
    }
  colsum += __shfl_xor(colsum, 32, 64);
  if (g == 0 && jv) X[(size_t)j * (DV + 1) + DV] = colsum;
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
  const dim3 xg((unsigned)(((a.r + XJG - 1) / XJG) * a.nchunk * a.H));
  if (a.n % 4 == 0 && a.chunk_rows % 4 == 0)
    hipLaunchKernelGGL((x_partial_kernel<TV, DV, true>), xg, dim3(64 * XW), 0, st, a);
  else
    hipLaunchKernelGGL((x_partial_kernel<TV, DV, false>), xg, dim3(64 * XW), 0, st, a);
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
  __shared__ int s_taken;
  __shared__ uint32_t s_fl;
  const int h = blockIdx.x, r = a.B * a.rb;
  if (threadIdx.x == 0) {
    s_taken = 0;
    s_fl = 0u;
  }
  for (int j = threadIdx.x; j < r; j += 256) {
    const int b = j / a.rb, sub = h * a.B + b;
    const int s = a.piv_sub[(size_t)sub * a.rb + j % a.rb];
    a.pivots[(size_t)h * r + j] = s >= 0 ? s + b * a.nb : -1;
  }
  // the bins' ranks and flags: one thread per bin, summed in LDS (an integer sum and an OR, so
  // the order does not matter)
  int taken = 0;
  uint32_t fl = 0u;
  for (int b = threadIdx.x; b < a.B; b += 256) {
    taken += a.rank_sub[h * a.B + b];
    fl |= a.flags_sub[h * a.B + b];
  }
  __syncthreads();
  if (taken) atomicAdd(&s_taken, taken);
  if (fl) atomicOr(&s_fl, fl);
  __syncthreads();
  if (threadIdx.x == 0) {
    a.rank[h] = s_taken;
    a.flags[h] = s_fl;
    a.rank_slots[h] = r;
  }
}

hipError_t launch_bins_combine(const BinsArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bins_combine_kernel, dim3(a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace wc
