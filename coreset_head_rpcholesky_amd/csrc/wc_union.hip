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

// sN[t][c] = G[t * ld + c] for a 64 x 64 block of a row-major matrix with ld % 4 == 0.
__device__ __forceinline__ void stage_direct(float (*sN)[kLP], const float* G, size_t ld) {
  const int tid = threadIdx.x, t = tid >> 2, c0 = 16 * (tid & 3);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<float4*>(&sN[t][c0 + 4 * q]) =
        *reinterpret_cast<const float4*>(G + (size_t)t * ld + c0 + 4 * q);
}

// x where keep holds, else +0 (also for a non-finite x), by a bit mask: no select that the
// compiler could turn into a branch around the load that produced x
__device__ __forceinline__ float keep_if(float x, bool keep) {
  return __uint_as_float(__float_as_uint(x) & (keep ? 0xffffffffu : 0u));
}

__device__ __forceinline__ void zero_acc(float acc[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = 0.f;
}

// ---- the slots of wc_weights_keys: pivots past the head's rank become empty (-1) -----------
__global__ void __launch_bounds__(256) union_mask_kernel(const int32_t* pivots, const int32_t* rank, int32_t* out,
                                                         int r) {
  const int h = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j < r) out[(size_t)h * r + j] = j < rank[h] ? pivots[(size_t)h * r + j] : -1;
}

// ---- gather: the coreset keys as rows, zero rows for empty slots ---------------------------
template <typename T, int D>
__global__ void __launch_bounds__(64) union_gather_kernel(UnionArgs a) {
  const int j = blockIdx.x, h = blockIdx.y;
  const int s = a.pivots[(size_t)h * a.r + j];
  const bool valid = s >= 0 && wc_index_ok(s, a.n, a.flags ? a.flags + h : nullptr);
  const T* K = reinterpret_cast<const T*>(a.K) + ((size_t)h * a.n + (valid ? s : 0)) * D;
  T* Qs = reinterpret_cast<T*>(a.Qs) + ((size_t)h * a.r + j) * D;
  for (int e = threadIdx.x; e < D; e += 64) Qs[e] = valid ? K[e] : T(0);
}

// ---- gram: A = exp(beta K_S K_S^T) on the lower blocks, its diagonal, zero X padding -------
// One workgroup per lower 64 x 64 block; the blocks of the heads go round-robin over the
// workgroups (consecutive workgroups land on different XCDs, so with 8 heads each XCD's L2
// holds one head's coreset keys).  bf16 keys: each wave forms a 32 x 32 quarter of the dot
// products on the bf16 matrix cores (the products of bf16 values are exact in fp32), its
// operands straight from global memory; fp32 keys: fp32 fused multiply-adds from LDS.
template <typename T, int D>
__global__ void __launch_bounds__(256) union_gram_kernel(UnionArgs a) {
  const int h = blockIdx.x % a.H, tid = threadIdx.x;
  int x = blockIdx.x / a.H, bi = 0;
  while (x > bi) x -= ++bi;
  const int bj = x;
  const T* Qs = reinterpret_cast<const T*>(a.Qs) + (size_t)h * a.r * D;
  float* A = a.A + (size_t)h * a.rp * a.rp;
  // slot validity, branch-free (the index clamped, so the load is always in bounds), so that all
  // of a thread's tests are requested together rather than one round trip per entry
  auto valid_at = [&](int j) {
    return (j < a.r) & (a.pivots[(size_t)h * a.r + min(j, a.r - 1)] >= 0);
  };
  auto finish = [&](int si, int sj, bool ok, float dot) {
    const float out = ok ? expf(a.beta * dot) : 0.f;
    if (bi == bj && si == sj) a.Hd[(size_t)h * a.rp + si] = out;
    return out;
  };
  if constexpr (sizeof(T) == 2) {
    const int lane = tid & 63, w = tid >> 6, g = lane >> 5;
    const int qm = 32 * (w >> 1), qn = 32 * (w & 1);
    // rows past r (padding slots) read row r-1 and are zeroed by finish()
    const int rm = min(bi * kUB + qm + (lane & 31), a.r - 1), rn = min(bj * kUB + qn + (lane & 31), a.r - 1);
    // lane l tests row qm + l % 32 of block bi and column qn + l % 32 of block bj; the rows'
    // results reach every lane by ballot (bit rho: row qm + rho)
    const bool vn = valid_at(bj * kUB + qn + (lane & 31));
    const uint64_t vrows = __ballot(valid_at(bi * kUB + qm + (lane & 31)));
    const bf16x8* pm = reinterpret_cast<const bf16x8*>(Qs + (size_t)rm * D + 8 * g);
    const bf16x8* pn = reinterpret_cast<const bf16x8*>(Qs + (size_t)rn * D + 8 * g);
    bf16x8 fm[D / 16], fn[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      fm[s] = pm[2 * s];
      fn[s] = pn[2 * s];
    }
    f32x16 c;
#pragma unroll
    for (int v = 0; v < 16; ++v) c[v] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) c = mfma32(fm[s], fn[s], c);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rho = 8 * (v >> 2) + 4 * g + (v & 3);
      const int si = bi * kUB + qm + rho, sj = bj * kUB + qn + (lane & 31);
      A[(size_t)si * a.rp + sj] = finish(si, sj, vn && ((vrows >> rho) & 1u), c[v]);
    }
  } else {
    __shared__ __attribute__((aligned(16))) float sI[32][kLP];
    __shared__ __attribute__((aligned(16))) float sJ[32][kLP];
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
    bool vi[4], vc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vi[i] = valid_at(bi * kUB + i0 + i);
      vc[i] = valid_at(bj * kUB + c0 + i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int si = bi * kUB + i0 + i;
      float out[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) out[c] = finish(si, bj * kUB + c0 + c, vi[i] && vc[c], acc[i][c]);
      *reinterpret_cast<float4*>(A + (size_t)si * a.rp + bj * kUB + c0) = make_float4(out[0], out[1], out[2], out[3]);
    }
  }
  if (blockIdx.x < (unsigned)a.H) {
    const int nc = a.dv + 1;
    float* X = a.X + (size_t)h * a.rp * nc;
    for (int e = a.r * nc + tid; e < a.rp * nc; e += 256) X[e] = 0.f;
  }
}

// ---- diag: M_kk = inverse of the Cholesky factor of the kept part of A_kk -------------------
// The workgroup eliminates the (already updated) block in sA with the leave-out rule, in two
// halves of 32 pivots on one wave joined by 32 x 32 products on the matrix cores
// (elim_block64_split, sS its scratch); left-out points of valid slots set WC_DFLAG_DEPENDENT.
// The diagonal entries H_jj (the scale of the leave-out test) are staged in LDS first.
__device__ __forceinline__ void diag_block(const UnionArgs& a, int h, int k, float (*sA)[kLP], float* sS,
                                           float (*sCol)[kUB], float* sHd) {
  if (threadIdx.x < kUB) sHd[threadIdx.x] = a.Hd[(size_t)h * a.rp + (size_t)k * kUB + threadIdx.x];
  const bool dependent = elim_block64_split<kLP>(&sA[0][0], sHd, a.tol, sS, sCol);
  store_block<kUB, kLP>(&sA[0][0], a.M + ((size_t)h * (a.rp / kUB) + k) * kUB * kUB);
  if (dependent && threadIdx.x == 0) atomicOr(&a.flags[h], WC_DFLAG_DEPENDENT);
}

// The first diagonal block (later ones are factored by the update of the step before).
__global__ void __launch_bounds__(256) union_diag0_kernel(UnionArgs a) {
  __shared__ __attribute__((aligned(16))) float sA[kUB][kLP];
  __shared__ __attribute__((aligned(16))) float sS[kUB][kLP];
  __shared__ __attribute__((aligned(16))) float sCol[2][kUB];
  __shared__ float sHd[kUB];
  const int h = blockIdx.x;
  const float* A = a.A + (size_t)h * a.rp * a.rp;
  stage_direct(sA, A, a.rp);
  __syncthreads();
  diag_block(a, h, 0, sA, &sS[0][0], sCol, sHd);
}

// ---- 32 x 32 products with the operands straight from global memory ----------------------
// One wave forms C = sum_t P[m][t] R[t][n] over t < 64 for a 32 x 32 tile on the fp32 matrix
// cores, in 32 steps of 32 x 32 x 2: lane l supplies P[l % 32][t] and R[t][l % 32] for the two
// values t of the step, and holds the result elements v = 0..15 at row 8 (v / 4) + 4 (l / 32) +
// v % 4, column l % 32.  Lane l takes t = 32 (l / 32) + s in step s for both operands (the 64
// terms in another order, the same sum), so that each lane reads 32 consecutive floats of a
// row-major operand row.
__device__ __forceinline__ int tile_row(int v) { return 8 * (v >> 2) + 4 * ((threadIdx.x >> 5) & 1) + (v & 3); }
__device__ __forceinline__ int tile_col() { return threadIdx.x & 31; }
// Element v of the lane's tile result in a row-major matrix with leading dimension ld: the
// lane's offset (one register) plus a part common to the wave.
__device__ __forceinline__ uint32_t tile_lane_off(uint32_t ld) {
  return 4 * ((threadIdx.x >> 5) & 1) * ld + (threadIdx.x & 31);
}
__device__ __forceinline__ uint32_t tile_v_off(int v, uint32_t ld) { return (uint32_t)(8 * (v >> 2) + (v & 3)) * ld; }
// Element `idx` (a 32-bit element offset) of the matrix at base, addressed as a byte offset
// from the wave's common base.
__device__ __forceinline__ float& at32(float* base, uint32_t idx) {
  return *reinterpret_cast<float*>(reinterpret_cast<char*>(base) + 4u * idx);
}

// f[s] = G[(l % 32) * ld + 32 (l / 32) + s]: 32 rows of a 64-wide block as the P operand (or
// as R transposed: R[t][n] = G[n][t]); ld % 4 == 0, G 16-byte aligned.
__device__ __forceinline__ void load_rows(float (&f)[32], const float* G, size_t ld) {
  const int lane = threadIdx.x & 63;
  const float4* p = reinterpret_cast<const float4*>(G + (size_t)(lane & 31) * ld + 32 * (lane >> 5));
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 v = p[q];
    f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
  }
}

// The L blocks in operand order.  The strictly upper 64 x 64 blocks of A are never used, so
// block (k, i) above the diagonal holds L_ik (i > k) a second time, arranged so that a wave
// reads the operand of a 32-row half with coalesced loads: element (rho, t) of half hh (row
// 32 hh + rho of L_ik, column t) sits at float f = 2048 hh + 256 (s / 4) + 4 lane + s % 4 with
// lane = rho + 32 (t / 32), s = t % 32, and float f of the block at row f / 64, column f % 64
// of block (k, i) of A.  Load q of a lane then reads 16 bytes of one of 4 consecutive 256-byte
// row pieces (8 cache lines per wave) instead of one of 64 rows (64 lines).
__device__ __forceinline__ float* frag_at(float* A, int rp, int k, int i, int f) {
  return A + (size_t)(k * kUB + (f >> 6)) * rp + (size_t)i * kUB + (f & 63);
}
// f[s] = rows 32 hh .. 32 hh + 31 of L_ik in the operand order of load_rows
__device__ __forceinline__ void load_frag(float (&f)[32], float* A, int rp, int k, int i, int hh) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(frag_at(A, rp, k, i, 2048 * hh + 256 * q + 4 * lane));
    f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
  }
}

// f[s] = G[(32 (l / 32) + s) * ld + col + l % 32], zero for columns at or past ncol: 32 columns
// of a 64-row block as the R operand.  The address is clamped, so every load is in bounds.
__device__ __forceinline__ void load_cols(float (&f)[32], const float* G, int ld, int col, int ncol) {
  const int lane = threadIdx.x & 63, c = col + (lane & 31);
  const bool ok = c < ncol;
  // byte offsets from the wave's common base: one register per lane, not one address per load
  const uint32_t off = 4u * ((uint32_t)(32 * (lane >> 5)) * ld + (ok ? c : ncol - 1));
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const char* base = reinterpret_cast<const char*>(G + (size_t)s * ld);   // common to the wave
    const float v = *reinterpret_cast<const float*>(base + off);
    f[s] = ok ? v : 0.f;
  }
}

__device__ __forceinline__ f32x16 mm32(const float (&fp)[32], const float (&fr)[32]) {
  f32x16 c;
#pragma unroll
  for (int v = 0; v < 16; ++v) c[v] = 0.f;
#pragma unroll
  for (int s = 0; s < 32; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(fp[s], fr[s], c, 0, 0, 0);
  return c;
}

// mm32 with mid() issued after the first 16 steps, when their operand registers are free (the
// loads of the block to be updated go there, so that they overlap the second half).
template <class F>
__device__ __forceinline__ f32x16 mm32_mid(const float (&fp)[32], const float (&fr)[32], F mid) {
  __builtin_amdgcn_sched_barrier(0);   // the operand loads all issued before the first product
  f32x16 c;
#pragma unroll
  for (int v = 0; v < 16; ++v) c[v] = 0.f;
#pragma unroll
  for (int s = 0; s < 16; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(fp[s], fr[s], c, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  mid();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 16; s < 32; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(fp[s], fr[s], c, 0, 0, 0);
  return c;
}

// ---- panel: L_ik = A_ik M_kk^T (i > k) and Z_k = M_kk X_k, in place ----------------------------
// One wave per item, so that every block a wave overwrites was read by that wave alone: a
// 32-row slice of some A_ik (both 32-column halves, P = its rows, R = M_kk^T), or a 32-column
// slice of X_k (both 32-row halves, P = rows of M_kk, R = those columns of X_k).  The items of
// the heads go round-robin over the workgroups.
__global__ void __launch_bounds__(64) union_panel_kernel(UnionArgs a, int k) {
  const int nb = a.rp / kUB, T = nb - k - 1, nc = a.dv + 1;
  const int h = blockIdx.x % a.H, x = blockIdx.x / a.H;
  const float* M = a.M + ((size_t)h * nb + k) * kUB * kUB;
  float* A = a.A + (size_t)h * a.rp * a.rp;
  float fp[32], fr[32], fq[32];
  f32x16 c0, c1;
  if (x < 2 * T) {
    float* Ls = A + ((size_t)(k + 1) * kUB + 32 * x) * a.rp + (size_t)k * kUB;   // rows 32 x of the panel
    load_rows(fp, Ls, a.rp);
    load_rows(fr, M, kUB);
    load_rows(fq, M + 32 * kUB, kUB);
    __builtin_amdgcn_sched_barrier(0);   // all operand loads in flight before the first product
    c0 = mm32(fp, fr);
    c1 = mm32(fp, fq);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      Ls[(size_t)tile_row(v) * a.rp + tile_col()] = c0[v];
      Ls[(size_t)tile_row(v) * a.rp + 32 + tile_col()] = c1[v];
    }
    // the operand-order copy in block (k, i): rows 32 (x % 2) .. of L_ik are half x % 2
    const int i = k + 1 + (x >> 1), hh = x & 1, n = tile_col();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rho = tile_row(v), fb = 2048 * hh + 256 * (n >> 2) + (n & 3);
      *frag_at(A, a.rp, k, i, fb + 4 * rho) = c0[v];
      *frag_at(A, a.rp, k, i, fb + 4 * (rho + 32)) = c1[v];
    }
  } else {
    const int col = 32 * (x - 2 * T);
    float* Xk = a.X + ((size_t)h * a.rp + (size_t)k * kUB) * nc;
    load_cols(fr, Xk, nc, col, nc);
    load_rows(fp, M, kUB);
    load_rows(fq, M + 32 * kUB, kUB);
    __builtin_amdgcn_sched_barrier(0);
    c0 = mm32(fp, fr);
    c1 = mm32(fq, fr);
    if (col + tile_col() < nc) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        Xk[(size_t)tile_row(v) * nc + col + tile_col()] = c0[v];
        Xk[(size_t)(32 + tile_row(v)) * nc + col + tile_col()] = c1[v];
      }
    }
  }
}

// ---- update: A_ij -= L_ik L_jk^T (k < j <= i), X_i -= L_ik Z_k --------------------------------
// A workgroup takes one 64 x 64 block, each wave a 32 x 32 quarter of it.  The first H
// workgroups take block (k+1, k+1) of each head: it has no other writer in this step, so its
// workgroup also factors it (diag_block for block column k+1) from LDS; that is the longest
// path of the step, so it starts first.  The other blocks go round-robin over the heads.
// Launch bounds of three workgroups per CU (up to 168 registers) rather than four (128), which
// measured about 25 us faster over the 31 update launches of r = 2048.
__global__ void __launch_bounds__(256, 3) union_update_kernel(UnionArgs a, int k) {
  __shared__ __attribute__((aligned(16))) float sA[kUB][kLP];
  __shared__ __attribute__((aligned(16))) float sS[kUB][kLP];
  __shared__ __attribute__((aligned(16))) float sCol[2][kUB];
  __shared__ float sHd[kUB];
  const int nb = a.rp / kUB, T = nb - k - 1, nc = a.dv + 1, nxz = (nc + kUB - 1) / kUB;
  const int npairs = T * (T + 1) / 2;
  int h, x;
  if ((int)blockIdx.x < a.H) {
    h = blockIdx.x;
    x = 0;
  } else {
    const int y = blockIdx.x - a.H;
    h = y % a.H;
    x = 1 + y / a.H;
  }
  const int w = threadIdx.x >> 6, qm = 32 * (w >> 1), qn = 32 * (w & 1);
  float* A = a.A + (size_t)h * a.rp * a.rp;
  float fp[32], fr[32];
  if (x < npairs) {
    int xx = x, ii = 0;
    while (xx > ii) xx -= ++ii;
    const int i = k + 1 + ii, j = k + 1 + xx;
    load_frag(fp, A, a.rp, k, i, qm >> 5);
    load_frag(fr, A, a.rp, k, j, qn >> 5);
    float* Aij = A + ((size_t)i * kUB + qm) * a.rp + (size_t)j * kUB + qn;
    const uint32_t lo = tile_lane_off(a.rp);
    float old[16];
    const f32x16 c = mm32_mid(fp, fr, [&] {
#pragma unroll
      for (int v = 0; v < 16; ++v) old[v] = at32(Aij + tile_v_off(v, a.rp), lo);
    });
    if (x == 0) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sA[qm + tile_row(v)][qn + tile_col()] = old[v] - c[v];
      diag_block(a, h, k + 1, sA, &sS[0][0], sCol, sHd);
      return;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) at32(Aij + tile_v_off(v, a.rp), lo) = old[v] - c[v];
  } else {
    const int y = x - npairs, i = k + 1 + y / nxz, col = (y % nxz) * kUB + qn;
    if (col >= nc) return;   // a quarter wholly past the last column
    float* X = a.X + (size_t)h * a.rp * nc;
    load_frag(fp, A, a.rp, k, i, qm >> 5);
    load_cols(fr, X + (size_t)k * kUB * nc, nc, col, nc);
    float* Xi = X + ((size_t)i * kUB + qm) * nc + col;
    const bool ok = col + tile_col() < nc;
    // clamped column: every load in bounds
    const uint32_t lo = tile_lane_off(nc) - tile_col() + (ok ? tile_col() : nc - 1 - col);
    float old[16];
    const f32x16 c = mm32_mid(fp, fr, [&] {
#pragma unroll
      for (int v = 0; v < 16; ++v) old[v] = at32(Xi + tile_v_off(v, nc), lo);
    });
    if (ok) {
#pragma unroll
      for (int v = 0; v < 16; ++v) at32(Xi + tile_v_off(v, nc), lo) = old[v] - c[v];
    }
  }
}

// ---- backward substitution, a range of block steps per launch ------------------------------
// The columns of W = L^{-T} Z are independent, so one workgroup takes kBackCols of them for one
// head and runs the block steps k = khi-1 .. klo of a range itself, the range's slice of Z
// resident in LDS:
//     W_k = M_kk^T Z_k,   then Z_j -= L_kj^T W_k for every klo <= j < k.
// The blocks below the range then take all of the range's W in one product
// (union_back_gemm_kernel) before the next range down, so that most of the work runs on the
// whole chip instead of on one workgroup per head and column slice.
// Products on the fp32 matrix cores, 16 x 16 x 4 (lane l: A[l % 16][l / 16], B[l / 16][l % 16],
// D rows 4 (l / 16) .. + 3 of column l % 16).  The A operands (M_kk and L_kj, read transposed)
// come straight from global memory, one step ahead of their products; the B operands (Z_k,
// W_k) from LDS.  Per step: waves 0-3 form the four 16-row tiles of W_k, then all waves share
// the 4 (k - klo) tiles of the update.  The slices of the heads go round-robin over the
// workgroups, so that with 8 heads the slices of one head share an XCD and its L2 copy of L.
constexpr int kBackCols = 16;
constexpr int kBackRange = 8;   // blocks per range: 512 rows x kBackCols floats of Z in LDS
constexpr int kBackWaves = 8;

__global__ void __launch_bounds__(64 * kBackWaves) union_back_slices_kernel(UnionArgs a, int klo, int khi) {
  __shared__ __attribute__((aligned(16))) float sZ[kBackRange * kUB][kBackCols];
  __shared__ __attribute__((aligned(16))) float sW[kUB][kBackCols];
  const int h = blockIdx.x % a.H, col0 = (blockIdx.x / a.H) * kBackCols, tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6, lr = lane & 15, lk = lane >> 4;
  const int nb = a.rp / kUB, nc = a.dv + 1, top = khi - 1;
  const float* Mh = a.M + (size_t)h * nb * kUB * kUB;
  const float* A = a.A + (size_t)h * a.rp * a.rp;
  const float* X = a.X + ((size_t)h * a.rp + (size_t)klo * kUB) * nc;
  float* W = a.W + (size_t)h * a.r * nc;
  {
    // the range's Z slice into LDS: a fixed number of unconditional (clamped) loads per thread,
    // all requested before the first LDS store
    constexpr int per = kBackRange * kUB * kBackCols / (64 * kBackWaves), step = 64 * kBackWaves / kBackCols;
    const int nrows = (khi - klo) * kUB, c = tid % kBackCols;
    const bool cok = col0 + c < nc;
    float z[per];
#pragma unroll
    for (int i = 0; i < per; ++i)
      z[i] = keep_if(X[(size_t)min(tid / kBackCols + step * i, nrows - 1) * nc + (cok ? col0 + c : nc - 1)], cok);
#pragma unroll
    for (int i = 0; i < per; ++i)
      if (tid / kBackCols + step * i < nrows) sZ[tid / kBackCols + step * i][c] = z[i];
  }
  // A operand of a 16-row tile: av[s] = G[(4 s + lk) * ld + lr], t = 4 s + lk the summed index
  auto load_a = [&](float (&av)[16], const float* G, size_t ld) {
#pragma unroll
    for (int s = 0; s < 16; ++s) av[s] = G[(size_t)(4 * s + lk) * ld + lr];
  };
  // update tile `tile` of step k: rows 16 (tile % 4) .. of block j = klo + tile / 4, L_kj read
  // transposed
  auto tile_src = [&](int k, int tile) {
    return A + (size_t)k * kUB * a.rp + (size_t)(klo + (tile >> 2)) * kUB + 16 * (tile & 3);
  };
  float am[16], at[16];
  if (wid < 4) load_a(am, Mh + (size_t)top * kUB * kUB + 16 * wid, kUB);
  if (wid < 4 * (top - klo)) load_a(at, tile_src(top, wid), a.rp);
  __syncthreads();
  for (int k = top; k >= klo; --k) {
    const int kl = k - klo;   // blocks of the range below block k
    if (wid < 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(am[s], sZ[kl * kUB + 4 * s + lk][lr], acc, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * wid + 4 * lk + v, wr = k * kUB + row;
        sW[row][lr] = acc[v];
        if (wr < a.r && col0 + lr < nc) W[(size_t)wr * nc + col0 + lr] = acc[v];
      }
      if (k > klo) load_a(am, Mh + (size_t)(k - 1) * kUB * kUB + 16 * wid, kUB);
    }
    __syncthreads();
    // (a wave without a tile in this step has none in the next either)
    for (int tile = wid; tile < 4 * kl; tile += kBackWaves) {
      float an[16];
      const int next = tile + kBackWaves;
      // the next tile of this step, or the first of the next step
      if (next < 4 * kl) load_a(an, tile_src(k, next), a.rp);
      else if (wid < 4 * (kl - 1)) load_a(an, tile_src(k - 1, wid), a.rp);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(at[s], sW[4 * s + lk][lr], acc, 0, 0, 0);
      const int r0 = (tile >> 2) * kUB + 16 * (tile & 3) + 4 * lk;
#pragma unroll
      for (int v = 0; v < 4; ++v) sZ[r0 + v][lr] -= acc[v];
#pragma unroll
      for (int s = 0; s < 16; ++s) at[s] = an[s];
    }
    __syncthreads();
  }
}

// Z_j -= sum over k in [klo, khi) of L_kj^T W_k for every block j < klo: the rows below a range
// take all of its weights in one product.  One workgroup per 32 x 32 tile of Z (rows row0 ..,
// columns col0 ..) of a head; each of its four waves sums a quarter of the range's rows on the
// fp32 matrix cores (32 x 32 x 2, lane l supplying L[kk][row0 + l % 32] and W[kk][col0 + l % 32]
// for the step's row kk = k0 + 2 s + l / 32; rows of W at or past r and columns past dv are
// zero), and the quarters are added through LDS in a fixed order.
__global__ void __launch_bounds__(256) union_back_gemm_kernel(UnionArgs a, int klo) {
  // a range with blocks below it is always a whole one (the ranges are cut from the top)
  constexpr int q = kBackRange * kUB / 4;   // range rows per wave
  constexpr int ng = q / 16;                // groups of 8 steps (16 rows)
  __shared__ float sC[3][16][64];
  const int nc = a.dv + 1, nct = (nc + 31) / 32;
  const int h = blockIdx.x % a.H, tile = blockIdx.x / a.H;
  const int row0 = (tile / nct) * 32, col0 = (tile % nct) * 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31;
  const int k0 = klo * kUB + w * q + (lane >> 5);
  const int c = col0 + l32;
  const bool cok = c < nc;
  const float* L = a.A + (size_t)h * a.rp * a.rp + row0 + l32;
  const float* Wc = a.W + (size_t)h * a.r * nc + (cok ? c : nc - 1);
  // the loads are unconditional (clamped row of W); rows at or past r and columns past dv are
  // zeroed at the point of use
  float pg[2][8], wg[2][8];
  auto load_group = [&](int grp, float (&pv)[8], float (&wv)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kk = k0 + 16 * grp + 2 * s;
      pv[s] = L[(size_t)kk * a.rp];
      wv[s] = Wc[(size_t)min(kk, a.r - 1) * nc];
    }
  };
  load_group(0, pg[0], wg[0]);
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int grp = 0; grp < ng; ++grp) {
    // scheduling fences: the next group's loads all go out before this group's products
    __builtin_amdgcn_sched_barrier(0);
    if (grp + 1 < ng) load_group(grp + 1, pg[(grp + 1) & 1], wg[(grp + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kk = k0 + 16 * grp + 2 * s;
      const float wv = keep_if(wg[grp & 1][s], cok && kk < a.r);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(pg[grp & 1][s], wv, acc, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (w > 0) {
#pragma unroll
    for (int v = 0; v < 16; ++v) sC[w - 1][v][lane] = acc[v];
  }
  __syncthreads();
  if (w > 0 || !cok) return;
  float* Z = a.X + ((size_t)h * a.rp + row0) * nc + c;
  float z[16];   // all of the tile's old values requested before the first store
#pragma unroll
  for (int v = 0; v < 16; ++v) z[v] = Z[(size_t)tile_row(v) * nc];
#pragma unroll
  for (int v = 0; v < 16; ++v)
    Z[(size_t)tile_row(v) * nc] = z[v] - (((acc[v] + sC[0][v][lane]) + sC[1][v][lane]) + sC[2][v][lane]);
}

template <typename T, int D>
hipError_t run_gather(const UnionArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((union_gather_kernel<T, D>), dim3(a.r, a.H), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_gram(const UnionArgs& a, hipStream_t st) {
  const int nb = a.rp / kUB;
  hipLaunchKernelGGL((union_gram_kernel<T, D>), dim3(a.H * (nb * (nb + 1) / 2)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_union_mask(const int32_t* pivots, const int32_t* rank, int32_t* out, int H, int r, hipStream_t st) {
  hipLaunchKernelGGL(union_mask_kernel, dim3((r + 255) / 256, H), dim3(256), 0, st, pivots, rank, out, r);
  return hipGetLastError();
}

hipError_t launch_union_gather(const UnionArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 64 ? run_gather<uint16_t, 64>(a, st) : run_gather<uint16_t, 128>(a, st);
  return a.d == 64 ? run_gather<float, 64>(a, st) : run_gather<float, 128>(a, st);
}

hipError_t launch_union_solve(const UnionArgs& a, hipStream_t st) {
  hipError_t e = a.bf16 ? (a.d == 64 ? run_gram<uint16_t, 64>(a, st) : run_gram<uint16_t, 128>(a, st))
                        : (a.d == 64 ? run_gram<float, 64>(a, st) : run_gram<float, 128>(a, st));
  if (e != hipSuccess) return e;
  const int nb = a.rp / kUB, nxz = (a.dv + 1 + kUB - 1) / kUB, nxs = (a.dv + 1 + 31) / 32;
  hipLaunchKernelGGL(union_diag0_kernel, dim3(a.H), dim3(256), 0, st, a);
  for (int k = 0; k < nb; ++k) {
    const int T = nb - k - 1;
    hipLaunchKernelGGL(union_panel_kernel, dim3(a.H * (2 * T + nxs)), dim3(64), 0, st, a, k);
    if (T > 0)
      hipLaunchKernelGGL(union_update_kernel, dim3(a.H * (T * (T + 1) / 2 + T * nxz)), dim3(256), 0, st, a, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return launch_union_back(a, st);
}

hipError_t launch_union_back(const UnionArgs& a, hipStream_t st) {
  const int nb = a.rp / kUB, ns = (a.dv + 1 + kBackCols - 1) / kBackCols, nct = (a.dv + 1 + 31) / 32;
  for (int khi = nb; khi > 0; khi -= kBackRange) {
    const int klo = khi > kBackRange ? khi - kBackRange : 0;
    hipLaunchKernelGGL(union_back_slices_kernel, dim3(ns * a.H), dim3(64 * kBackWaves), 0, st, a, klo, khi);
    if (klo > 0)
      hipLaunchKernelGGL(union_back_gemm_kernel, dim3(a.H * 2 * klo * nct), dim3(256), 0, st, a, klo);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wc
