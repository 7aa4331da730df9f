// Attention of every query over the weighted coreset (page gptget.net/papers/2602.10056,
// Abstract: attend only over a small weighted coreset; gist.science/de/paper/2602.10056,
// "Methodik" part 2: the output is formed from the r coreset elements alone):
//     Y = exp(beta Q K_S^T) W,   O = Y[:, :dv] / Y[:, dv].
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, one wave = 32 queries):
//   scores   S^T (32 coreset x 32 queries) = K_S Q^T, K_S chunk staged in LDS, Q^T as the
//            B operand straight from the query rows;
//   values   Y^T (32 value columns x 32 queries) += W^T P^T.  The accumulator of the score
//            MFMA holds, in lane l, coreset rows 8(v/4) + 4(l/32) + v%4 of query l%32; packed
//            to bf16 it is directly the B operand of the value MFMA provided W^T's columns
//            (coreset index) are stored in the matching permuted order (perm32).
//   normaliser Y[:, dv] on the vector units: for bf16 inputs, packed bf16 dot products of the
//            same bf16-rounded P as the values with W[:, dv] rounded to bf16 (fp32 sums); for
//            fp32 inputs, fp32 products of P with the fp32 W[:, dv].  In bf16 each of P and
//            W[:, dv] carries a relative rounding of at most 2^-9, so a row whose normaliser
//            condition sum |P| |W[:, dv]| / |Y[:, dv]| is kappa has a normaliser error of at most
//            about 2^-8 kappa relative.
// No row-max shift is needed: any per-row factor cancels in the ratio, and the inputs are
// bounded.  fp32 inputs use hi + lo bf16 splits (three products per MFMA step).
#include "wc_device.h"
#include "wc_kernels.h"

namespace wc {

__device__ __forceinline__ int perm32_a(int j) {
  const int jb = j & ~31, jj = j & 31;
  const int qq = jj >> 4, rem = jj & 15;
  const int g = (rem & 7) >> 2, e = ((rem >> 3) << 2) | (rem & 3);
  return jb + 16 * qq + 8 * g + e;
}

__device__ __forceinline__ uint16_t bf16_bits(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }

// Tile-major layouts of the staged operands, per head.  K_S is cut into 64-row chunks, each an
// array [D/8][64 rows][8] of bf16: a chunk is one contiguous block, and the 16-byte pieces that
// 64 consecutive lanes need for one MFMA operand (same 8 columns, consecutive rows) are
// consecutive.  W^T (value column cc, permuted coreset position p) likewise, with chunks of 64
// positions stored as [8][DV][8].
__device__ __forceinline__ size_t ks_index(int j, int e, int D) {
  return ((size_t)((j >> 6) * (D / 8) + (e >> 3)) * 64 + (j & 63)) * 8 + (e & 7);
}
__device__ __forceinline__ size_t wt_index(int cc, int p, int DV) {
  return ((size_t)((p >> 6) * 8 + ((p & 63) >> 3)) * DV + cc) * 8 + (p & 7);
}

template <typename T, int D, int DV>
__global__ void __launch_bounds__(128) attend_prep_kernel(AttendArgs a) {
  constexpr bool SPLIT = sizeof(T) == 4;
  const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int rp = staged_rows(a);
  // slots past the rank, and slots a bin left empty (pivot -1), carry zero weight
  const int rk = a.rank[h];
  const int sj = j < rk ? a.pivots[(size_t)h * a.r + j] : -1;
  const bool valid = sj >= 0 && wc_index_ok(sj, a.n, a.flags ? a.flags + h : nullptr);
  const int s = valid ? sj : 0;
  const T* K = reinterpret_cast<const T*>(a.K) + ((size_t)h * a.n + s) * D;
  for (int e = tid; e < D; e += 128) {
    const float v = valid ? ld_elem<T>(K + e) : 0.f;
    __bf16 hi, lo;
    split_bf16(v, hi, lo);
    const size_t o = (size_t)h * rp * D + ks_index(j, e, D);
    a.KSh[o] = bf16_bits(hi);
    if (SPLIT) a.KSl[o] = bf16_bits(lo);
  }
  const int p = perm32_a(j);
  const float* W = a.W + ((size_t)h * a.r + (valid ? j : 0)) * (DV + 1);
  for (int c = tid; c < DV; c += 128) {
    const float w = valid ? W[c] : 0.f;
    __bf16 hi, lo;
    split_bf16(w, hi, lo);
    const size_t o = (size_t)h * DV * rp + wt_index(c, p, DV);
    a.Wph[o] = bf16_bits(hi);
    if (SPLIT) a.Wpl[o] = bf16_bits(lo);
  }
  if (tid == 0) {
    const float wd = valid ? W[DV] : 0.f;
    a.Wden[(size_t)h * rp + j] = wd;
    a.Wdh[(size_t)h * rp + p] = bf16_bits((__bf16)wd);
  }
}

// Inverse of perm32_a: the coreset row stored at permuted position p.
__device__ __forceinline__ int perm32_inv(int p) {
  const int pb = p & ~31, pp = p & 31;
  const int qq = pp >> 4, g = (pp >> 3) & 1, e = pp & 7;
  return pb + 16 * qq + (((e >> 2) << 3) | (g << 2) | (e & 3));
}

// Every key as a coreset row (row j = key j, rows past n zero) with W = [V, 1]: the staged
// operands of Y = exp(beta Q K^T) [V, 1].  One workgroup per 64-row chunk: the chunk's keys,
// then its values, are read with 16-byte loads into LDS and written out in the tile-major
// order of K_S and the permuted order of W^T, with contiguous 16-byte stores.
template <typename T, int D, int DV>
__global__ void __launch_bounds__(256) attend_prep_keys_kernel(AttendArgs a) {
  constexpr bool SPLIT = sizeof(T) == 4;
  constexpr int E = 16 / (int)sizeof(T);           // input elements per 16-byte load
  constexpr int W = (D > DV ? D : DV) + E;         // LDS row pitch (elements of T)
  __shared__ __attribute__((aligned(16))) T sX[64 * W];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int rp = staged_rows(a);
  const int j0 = c * 64;
  // keys (none with KSh NULL: the attention then reads the bf16 keys in place)
  if (a.KSh) {
    for (int e = tid; e < 64 * D / E; e += 256) {
      const int row = e / (D / E), col = (e % (D / E)) * E, j = j0 + row;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (j < a.n) v = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.K) + ((size_t)h * a.n + j) * D + col);
      *reinterpret_cast<uint4*>(&sX[row * W + col]) = v;
    }
    __syncthreads();
    const size_t kbase = (size_t)h * rp * D + (size_t)j0 * D;
    for (int u = tid; u < 64 * (D / 8); u += 256) {   // output unit (column group u / 64, row u % 64)
      const int cg = u >> 6, row = u & 63;
      if constexpr (!SPLIT) {
        *reinterpret_cast<uint4*>(a.KSh + kbase + 8 * (size_t)u) = *reinterpret_cast<const uint4*>(&sX[row * W + 8 * cg]);
        continue;
      }
      bf16x8 hi8, lo8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hi, lo;
        split_bf16(ld_elem<T>(&sX[row * W + 8 * cg + e]), hi, lo);
        hi8[e] = hi;
        lo8[e] = lo;
      }
      *reinterpret_cast<bf16x8*>(a.KSh + kbase + 8 * (size_t)u) = hi8;
      *reinterpret_cast<bf16x8*>(a.KSl + kbase + 8 * (size_t)u) = lo8;
    }
    __syncthreads();
  }
  // values
  for (int e = tid; e < 64 * DV / E; e += 256) {
    const int row = e / (DV / E), col = (e % (DV / E)) * E, j = j0 + row;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (j < a.n) v = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.V) + ((size_t)h * a.n + j) * DV + col);
    *reinterpret_cast<uint4*>(&sX[row * W + col]) = v;
  }
  __syncthreads();
  const size_t wbase = (size_t)h * DV * rp + (size_t)c * 64 * DV;
  for (int u = tid; u < 8 * DV; u += 256) {         // output unit (8 permuted positions, one column)
    const int grp = u / DV, col = u % DV;
    bf16x8 hi8, lo8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 hi, lo;
      split_bf16(ld_elem<T>(&sX[perm32_inv(8 * grp + e) * W + col]), hi, lo);
      hi8[e] = hi;
      lo8[e] = lo;
    }
    *reinterpret_cast<bf16x8*>(a.Wph + wbase + 8 * (size_t)u) = hi8;
    if (SPLIT) *reinterpret_cast<bf16x8*>(a.Wpl + wbase + 8 * (size_t)u) = lo8;
  }
  if (tid < 64) {
    const int j = j0 + tid;
    const float wd = j < a.n ? 1.f : 0.f;
    a.Wden[(size_t)h * rp + j] = wd;
    a.Wdh[(size_t)h * rp + perm32_a(j)] = bf16_bits((__bf16)wd);
  }
}

// Exact rows: row row0 + j of the staged layout holds key j of K with weights [v_j, 1]
// (j < n), so that its contribution is that of exact softmax attention.
template <typename T, int D, int DV>
__global__ void __launch_bounds__(128) attend_append_kernel(AttendArgs a) {
  constexpr bool SPLIT = sizeof(T) == 4;
  const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int rp = staged_rows(a), row = a.row0 + j;
  const T* K = reinterpret_cast<const T*>(a.K) + ((size_t)h * a.n + j) * D;
  const T* V = reinterpret_cast<const T*>(a.V) + ((size_t)h * a.n + j) * DV;
  for (int e = tid; e < D; e += 128) {
    __bf16 hi, lo;
    split_bf16(ld_elem<T>(K + e), hi, lo);
    const size_t o = (size_t)h * rp * D + ks_index(row, e, D);
    a.KSh[o] = bf16_bits(hi);
    if (SPLIT) a.KSl[o] = bf16_bits(lo);
  }
  const int p = perm32_a(row);
  for (int c = tid; c < DV; c += 128) {
    __bf16 hi, lo;
    split_bf16(ld_elem<T>(V + c), hi, lo);
    const size_t o = (size_t)h * DV * rp + wt_index(c, p, DV);
    a.Wph[o] = bf16_bits(hi);
    if (SPLIT) a.Wpl[o] = bf16_bits(lo);
  }
  if (tid == 0) {
    a.Wden[(size_t)h * rp + row] = 1.f;
    a.Wdh[(size_t)h * rp + p] = bf16_bits((__bf16)1.f);
  }
}

// Row q of head h of the unnormalised output (fp32, dv + 1 columns).
__device__ __forceinline__ float* yout_row(const AttendArgs& a, int h, int q) {
  return a.Yout + ((size_t)h * a.yrows + q) * (a.dv + 1);
}

template <typename T, int D, int DV>
__global__ void __launch_bounds__(256) attend_kernel(AttendArgs a) {
  constexpr bool SPLIT = sizeof(T) == 4;
  constexpr int KP = D + 8, WP = 32 + 8, NCT = DV / 32;
  __shared__ __attribute__((aligned(16))) __bf16 sKh[32 * KP];
  __shared__ __attribute__((aligned(16))) __bf16 sKl[SPLIT ? 32 * KP : 8];
  __shared__ __attribute__((aligned(16))) __bf16 sWh[DV * WP];
  __shared__ __attribute__((aligned(16))) __bf16 sWl[SPLIT ? DV * WP : 8];
  __shared__ float sWd[32];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y, sp = blockIdx.z;
  const int m = a.m, rp = staged_rows(a), nchk = scanned_rows(a) / 32;
  // rows at or past the scan bound carry no weight even when the staged row is not zero
  const int lim = a.scan_rows ? a.scan_rows : rp;
  const int q = blockIdx.x * 128 + wid * 32 + l32;
  const bool qv = q < m;
  const float bl2e = a.beta_log2e;
  const T* Q = reinterpret_cast<const T*>(a.Q) + (size_t)h * m * D;

  bf16x8 qh[D / 16], ql[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = qv ? ld_elem<T>(Q + (size_t)q * D + 16 * kk + 8 * g + e) : 0.f;
      __bf16 hi, lo;
      split_bf16(v, hi, lo);
      qh[kk][e] = hi;
      ql[kk][e] = lo;
    }
  f32x16 y[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) y[ct][v] = 0.f;
  float den = 0.f;
  const int per = (nchk + a.nsplit - 1) / a.nsplit;
  const int cb = sp * per, ce = min(nchk, cb + per);
  const uint16_t* KSh = a.KSh + (size_t)h * rp * D;
  const uint16_t* KSl = a.KSl ? a.KSl + (size_t)h * rp * D : nullptr;
  const uint16_t* Wph = a.Wph + (size_t)h * DV * rp;
  const uint16_t* Wpl = a.Wpl ? a.Wpl + (size_t)h * DV * rp : nullptr;
  for (int c = cb; c < ce; ++c) {
    __syncthreads();
    for (int e = tid; e < 32 * (D / 8); e += 256) {
      const int jj = e / (D / 8), k8 = e % (D / 8);
      const size_t src = ks_index(c * 32 + jj, 8 * k8, D);
      *reinterpret_cast<uint4*>(sKh + jj * KP + 8 * k8) = *reinterpret_cast<const uint4*>(KSh + src);
      if (SPLIT) *reinterpret_cast<uint4*>(sKl + jj * KP + 8 * k8) = *reinterpret_cast<const uint4*>(KSl + src);
    }
    for (int e = tid; e < DV * 4; e += 256) {
      const int cc = e / 4, k8 = e % 4;
      const size_t src = wt_index(cc, c * 32 + 8 * k8, DV);
      *reinterpret_cast<uint4*>(sWh + cc * WP + 8 * k8) = *reinterpret_cast<const uint4*>(Wph + src);
      if (SPLIT) *reinterpret_cast<uint4*>(sWl + cc * WP + 8 * k8) = *reinterpret_cast<const uint4*>(Wpl + src);
    }
    if (tid < 32) sWd[tid] = a.Wden[(size_t)h * rp + c * 32 + tid];
    __syncthreads();
    f32x16 sc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 kh = *reinterpret_cast<const bf16x8*>(sKh + l32 * KP + 16 * kk + 8 * g);
      sc = mfma32(kh, qh[kk], sc);
      if (SPLIT) {
        const bf16x8 kl = *reinterpret_cast<const bf16x8*>(sKl + l32 * KP + 16 * kk + 8 * g);
        sc = mfma32(kh, ql[kk], sc);
        sc = mfma32(kl, qh[kk], sc);
      }
    }
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int jj = 8 * (v >> 2) + 4 * g + (v & 3);
      const float p = c * 32 + jj < lim ? __builtin_amdgcn_exp2f(sc[v] * bl2e) : 0.f;
      den = fmaf(p, sWd[jj], den);
      __bf16 hi, lo;
      split_bf16(p, hi, lo);
      ph[v >> 3][v & 7] = hi;
      pl[v >> 3][v & 7] = lo;
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const bf16x8 wh = *reinterpret_cast<const bf16x8*>(sWh + (ct * 32 + l32) * WP + 16 * qq + 8 * g);
        y[ct] = mfma32(wh, ph[qq], y[ct]);
        if (SPLIT) {
          const bf16x8 wl = *reinterpret_cast<const bf16x8*>(sWl + (ct * 32 + l32) * WP + 16 * qq + 8 * g);
          y[ct] = mfma32(wh, pl[qq], y[ct]);
          y[ct] = mfma32(wl, ph[qq], y[ct]);
        }
      }
  }
  den += __shfl_xor(den, 32, 64);
  if (a.nsplit == 1 && a.Yout) {
    if (!qv) return;
    float* Y = yout_row(a, h, q);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) Y[ct * 32 + 8 * (v >> 2) + 4 * g + (v & 3)] = y[ct][v];
    if (g == 0) Y[DV] = den;
  } else if (a.nsplit == 1) {
    if (!qv) return;
    if (!(den > 0.f)) atomicOr(&a.flags[h], WC_DFLAG_DENOM);
    const float inv = 1.0f / den;
    T* O = reinterpret_cast<T*>(a.O) + ((size_t)h * m + q) * DV;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int col = ct * 32 + 8 * v4 + 4 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) st_elem<T>(O + col + e, y[ct][4 * v4 + e] * inv);
      }
  } else {
    if (!qv) return;
    float* Yp = a.Ypart + (((size_t)h * a.nsplit + sp) * m + q) * (DV + 1);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) Yp[ct * 32 + 8 * (v >> 2) + 4 * g + (v & 3)] = y[ct][v];
    if (g == 0) Yp[DV] = den;
  }
}

// bf16 inputs.  A workgroup takes 256 queries (kAttendWaves waves of kAttendNQ x 32).  The
// coreset is walked in 64-row chunks through a ring of LDS buffers filled by direct
// global-to-LDS loads (no staging registers, no LDS store instructions): while chunk c is in
// use, chunk c+1 is resident and the next ones are loading, so one barrier per chunk is the
// only synchronisation.  With the tile-major layouts above a chunk is copied as is, and the operand
// reads of consecutive lanes hit consecutive 16-byte units (no bank conflicts).
typedef __attribute__((address_space(3))) void* lds_void;

#ifndef WC_ATTEND_NQ
#define WC_ATTEND_NQ 1
#endif
constexpr int kAttendNQ = WC_ATTEND_NQ;          // groups of 32 queries per wave
constexpr int kAttendWaves = 8 / kAttendNQ;      // waves per workgroup
constexpr int kAttendQueries = 256;              // queries per workgroup
#ifndef WC_ATTEND_PREFETCH
#define WC_ATTEND_PREFETCH 2
#endif
constexpr int kAttendPrefetch = WC_ATTEND_PREFETCH;  // LDS operand reads run this many MFMAs of their kind ahead

template <int D, int DV>
struct AttendChunk {
  uint4 k[64 * D / 8];   // K_S chunk, [D/8][64][8] bf16
  uint4 w[DV * 64 / 8];  // W^T chunk, [8][DV][8] bf16
  uint4 wd[8];           // W[:, dv] in bf16, permuted like the columns of W^T
};

// One direct load: 16 bytes per lane from gptr into LDS at lds + 16 * lane.  Written as an asm
// statement so the compiler adds no wait of its own between the load and later LDS reads of
// other buffers (it cannot tell the buffers apart); the loads are waited for explicitly
// (vmcnt(0), then a barrier) before their buffer is read.  The statement has no register
// outputs, and its address operand is consumed when the instruction issues.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds) : "memory", "m0");
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), as an immediate the compiler's
// own wait tracking understands
constexpr int kVmcnt0 = 0x0F70;
#ifndef WC_ATTEND_RING
#define WC_ATTEND_RING 4
#endif
constexpr int kAttendRing = WC_ATTEND_RING;
// tiles of at least this many chunks take the deferred tile-end schedule (MODE 5, MODE 6)
constexpr int kAttendLongTile = 6;  // LDS chunk buffers: chunks in use, resident, loading
static_assert(kAttendRing == 3 || kAttendRing == 4, "ring of three or four chunks");
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void)const_cast<void*>(p);
}

// Wait until at most `pending` chunks of this wave's direct loads are still in flight (loads
// complete in order, so every older chunk has landed).  A chunk is KI + WI load instructions
// per wave, plus the normaliser column's on wave 0.
// s_waitcnt immediate for vmcnt <= n (6-bit count: low bits [3:0], high bits [15:14]).
constexpr int vmcnt_imm(int n) { return kVmcnt0 | (n & 15) | ((n >> 4) & 3) << 14; }

// EXTRA: further loads of this wave issued after those chunks (the next tile's query fragments)
// that may stay in flight too.
template <int D, int DV, int EXTRA = 0>
__device__ __forceinline__ void attend_wait(int pending, int wid) {
  constexpr int per = D / (8 * kAttendWaves) + DV / (8 * kAttendWaves);
  static_assert(2 * per + 2 + EXTRA < 64, "vmcnt field");
  if (pending <= 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(EXTRA));
  } else if (pending == 1) {
    if (wid == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(per + 1 + EXTRA));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(per + EXTRA));
  } else {
    if (wid == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * per + 2 + EXTRA));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * per + EXTRA));
  }
}

// KROW: the coreset rows are the rows of a row-major key matrix K with nrm rows (the all-keys
// pass, bf16 keys), read in place of a staged copy: lane l loads row 64 c + l (the last row for
// rows past nrm, which carry zero weight) at the instruction's column group, so that the chunk
// lands in LDS in the same [D/8][64][8] order.  Otherwise K is the staged layout.
template <int D, int DV, bool KROW>
__device__ __forceinline__ void attend_issue(AttendChunk<D, DV>& b, const uint16_t* K, int nrm, const uint16_t* Wph,
                                             const uint16_t* Wdh, int c, int wid, int lane) {
  constexpr int KI = D / (8 * kAttendWaves), WI = DV / (8 * kAttendWaves);  // 1 KB wave instructions per tile
  const char* wbase = reinterpret_cast<const char*>(Wph) + (size_t)c * 64 * DV * 2;
  const uint32_t lo = 16 * lane;
  if constexpr (KROW) {
    const char* krow = reinterpret_cast<const char*>(K) + (size_t)min(c * 64 + lane, nrm - 1) * D * 2;
#pragma unroll
    for (int i = 0; i < KI; ++i)
      dma16(krow + 16 * (kAttendWaves * i + wid), lds_addr(&b.k[64 * (kAttendWaves * i + wid)]));
  } else {
    const char* kbase = reinterpret_cast<const char*>(K) + (size_t)c * 64 * D * 2;
#pragma unroll
    for (int i = 0; i < KI; ++i)
      dma16(kbase + 1024 * (kAttendWaves * i + wid) + lo, lds_addr(&b.k[64 * (kAttendWaves * i + wid)]));
  }
#pragma unroll
  for (int i = 0; i < WI; ++i)
    dma16(wbase + 1024 * (kAttendWaves * i + wid) + lo, lds_addr(&b.w[64 * (kAttendWaves * i + wid)]));
  if (wid == 0 && lane < 32) dma4(Wdh + c * 64 + 2 * lane, lds_addr(&b.wd[0]));
}

// One pipeline step of one wave (NQ groups of 32 queries) at coreset unit u (32 rows): the
// scores of unit u+1 and the values of unit u-1 on the matrix cores, and the exponentials of
// unit u on the vector units, one score per group per MFMA slot, so both kinds of work are
// always available to issue.  Each LDS operand fragment feeds the NQ query groups; it is read
// kAttendPrefetch MFMA slots of its kind ahead, and scheduling fences hold this order.
template <int D, int DV, int NQ>
__device__ __forceinline__ void attend_step(const AttendChunk<D, DV>& bS, int uS, const AttendChunk<D, DV>& bE,
                                            int uE, const AttendChunk<D, DV>& bP, int uP,
                                            const bf16x8 (&qb)[NQ][D / 16], f32x16 (&y)[NQ][DV / 32],
                                            float (&den)[NQ][4], const f32x16 (&sc_cur)[NQ], f32x16 (&sc_next)[NQ],
                                            const bf16x8 (&pb_prev)[NQ][2], bf16x8 (&pb_cur)[NQ][2], int g, int l32) {
  constexpr int NK = D / 16, NW = DV / 16, NS = NK + NW;
  auto kfrag = [&](int kk) { return __builtin_bit_cast(bf16x8, bS.k[(2 * kk + g) * 64 + 32 * uS + l32]); };
  auto wfrag = [&](int i) {  // i = 2 ct + qq
    return __builtin_bit_cast(bf16x8, bP.w[(4 * uP + 2 * (i & 1) + g) * DV + 32 * (i >> 1) + l32]);
  };
  // W[:, dv] for the two halves of this lane's probabilities, in the same (permuted) order
  bf16x8 wd[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) wd[qq] = __builtin_bit_cast(bf16x8, bE.wd[4 * uE + 2 * qq + g]);
  bf16x8 kf[NK], wf[NW];
#pragma unroll
  for (int i = 0; i < kAttendPrefetch; ++i) {
    if (i < NK) kf[i] = kfrag(i);
    if (i < NW) wf[i] = wfrag(i);
  }
#pragma unroll
  for (int s = 0; s < NQ; ++s) sc_next[s] = f32x16{};
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int si = j * NK / NS;  // S slots before slot j
    if ((j + 1) * NK / NS > si) {
#pragma unroll
      for (int s = 0; s < NQ; ++s) sc_next[s] = mfma32(kf[si], qb[s][si], sc_next[s]);
      if (si + kAttendPrefetch < NK) kf[si + kAttendPrefetch] = kfrag(si + kAttendPrefetch);
    } else {
      const int i = j - si;
#pragma unroll
      for (int s = 0; s < NQ; ++s) y[s][i >> 1] = mfma32(wf[i], pb_prev[s][i & 1], y[s][i >> 1]);
      if (i + kAttendPrefetch < NW) wf[i + kAttendPrefetch] = wfrag(i + kAttendPrefetch);
    }
#pragma unroll
    for (int v = j * 16 / NS; v < (j + 1) * 16 / NS; ++v)
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        // the queries carry the factor beta log2(e), so the score is already a base-2 exponent
        pb_cur[s][v >> 3][v & 7] = (__bf16)__builtin_amdgcn_exp2f(sc_cur[s][v]);
        if (v & 1) {  // normaliser: packed bf16 products, the same rounded P and W as the values
          const bf16x2 pp = {pb_cur[s][v >> 3][(v & 7) - 1], pb_cur[s][v >> 3][v & 7]};
          const bf16x2 ww = {wd[v >> 3][(v & 7) - 1], wd[v >> 3][v & 7]};
          den[s][(v >> 1) & 3] = __builtin_amdgcn_fdot2_f32_bf16(pp, ww, den[s][(v >> 1) & 3], false);
        }
      }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The probabilities and normaliser sums of a pipeline step, pinned where the step ends: an
// empty asm statement that reads them keeps the compiler from sinking their exponentials past
// the chunk's waits and barrier into the next step (which would run them as one burst with
// the matrix cores idle instead of one per MFMA slot).
template <int NQ>
__device__ __forceinline__ void attend_pin(const bf16x8 (&pb)[NQ][2], const float (&den)[NQ][4]) {
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    asm volatile("" ::"v"(pb[s][0]), "v"(pb[s][1]));
    asm volatile("" ::"v"(den[s][0]), "v"(den[s][1]), "v"(den[s][2]), "v"(den[s][3]));
  }
}

// Scores of one 32-row unit whose rows from `left` on lie past the scan bound: set to -inf, so
// that their probabilities are exactly zero (row of accumulator entry v: 8(v/4) + 4g + v%4).
template <int NQ>
__device__ __forceinline__ void attend_mask(f32x16 (&sc)[NQ], int left, int g) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const bool out = 8 * (v >> 2) + 4 * g + (v & 3) >= left;
#pragma unroll
    for (int s = 0; s < NQ; ++s)
      if (out) sc[s][v] = -__builtin_inff();
  }
}

// The work of the attention is a list of tiles: (query tile of 256 queries, head, coreset split),
// query tile fastest, then split, then head.  The kernel is persistent: a grid of one workgroup
// per compute unit walks its tiles one after the other, and the coreset chunks of consecutive
// tiles form one stream through the LDS ring, so the loads of the next tile's first chunks and
// its query fragments overlap the end of the current tile instead of a new workgroup starting
// cold.  Workgroups are dealt to the 8 XCDs round-robin by id; when the counts allow, the
// workgroups of one XCD take a contiguous range of tiles, so a head's coreset is read through
// one or two XCDs' L2 instead of all eight.
struct AttendTile {
  int qt, h, sp, c0, nc;
};

__device__ __forceinline__ AttendTile attend_tile_at(const AttendArgs& a, int t, int QT, int nchk, int per) {
  AttendTile x;
  x.qt = t % QT;
  const int hs = t / QT;
  x.h = hs / a.nsplit;
  x.sp = hs % a.nsplit;
  x.c0 = x.sp * per;
  x.nc = min(nchk, x.c0 + per) - x.c0;
  return x;
}

// Index of this workgroup's j-th tile, or -1 past its last.
__device__ __forceinline__ int attend_wg_tile(int j, int T) {
  const int G = gridDim.x, b = blockIdx.x;
  if (T % 8 == 0 && G % 8 == 0) {
    const int per_xcd = G / 8, k = b / 8 + j * per_xcd;
    return k < T / 8 ? (b % 8) * (T / 8) + k : -1;
  }
  const int t = b + j * G;
  return t < T ? t : -1;
}

// Query fragments of 32 NQ queries of one tile, raw bf16.  Exactly NQ * D/16 load instructions
// per lane whatever the tile (rows past the last query read the last query's row, and are zeroed
// when scaled), so that the chunk waits can count them.
template <int D, int NQ>
__device__ __forceinline__ void attend_load_q(const AttendArgs& a, int h, int q0, int g, bf16x8 (&raw)[NQ][D / 16]) {
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.Q) + (size_t)h * a.m * D;
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    const int q = min(q0 + 32 * s, a.m - 1);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      raw[s][kk] = *reinterpret_cast<const bf16x8*>(Q + (size_t)q * D + 16 * kk + 8 * g);
  }
}

// The B operands of the score MFMA: query fragments scaled by beta log2(e) (one bf16 rounding,
// relative 2^-9 per element), so that the score is already a base-2 exponent; zero for rows
// past the last query.
template <int D, int NQ>
__device__ __forceinline__ void attend_scale_q(const bf16x8 (&raw)[NQ][D / 16], int q0, int m, float bl2e,
                                               bf16x8 (&qb)[NQ][D / 16]) {
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    const float f = q0 + 32 * s < m ? bl2e : 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[s][kk][e] = (__bf16)((float)raw[s][kk][e] * f);
  }
}

// The scaled query fragments, pinned where they are formed: an empty asm statement that reads
// them keeps the compiler from sinking the scaling (and the waits for the raw fragments in
// front of it) past the chunk loads issued next, where those waits would also cover the loads
// just issued.
template <int D, int NQ>
__device__ __forceinline__ void attend_pin_q(const bf16x8 (&qb)[NQ][D / 16]) {
#pragma unroll
  for (int s = 0; s < NQ; ++s)
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" ::"v"(qb[s][kk]));
}

// MASK: the scan bound falls inside a 128-row block (a cache decoded over a prefix of its
// rows), so the units that cross it are masked; without it every scanned row counts.
// KROW: the coreset rows are the bf16 keys K themselves, read in place (attend_issue).
template <int D, int DV, bool MASK, bool KROW>
__global__ void __launch_bounds__(64 * kAttendWaves) __attribute__((amdgpu_waves_per_eu(kAttendWaves / 4, kAttendWaves / 4)))
attend_bf16_kernel(AttendArgs a) {
  constexpr int NK = D / 16, NW = DV / 16, NCT = DV / 32, NQ = kAttendNQ, R = kAttendRing, QN = NQ * NK;
  __shared__ AttendChunk<D, DV> sb[R];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = a.m, rp = staged_rows(a);
  const float bl2e = a.beta_log2e;
  const int QT = (m + kAttendQueries - 1) / kAttendQueries, T = QT * a.H * a.nsplit;
  const int nchk = scanned_rows(a) / 64, per = (nchk + a.nsplit - 1) / a.nsplit;
  // rows at or past the scan bound carry no weight even when the staged row is not zero: the
  // scores of a unit that crosses it are set to -inf before they are exponentiated
  const int lim = a.scan_rows ? a.scan_rows : rp;
  const int qoff = wid * 32 * NQ + l32;

  // chunk loads run R-1 chunks ahead of the computation, through the tiles in order: the issue
  // cursor is (tile ij, chunk ic of it); `issued` counts the chunks issued so far
  int ij = 0, ic = 0, issued = 0;
  int it = attend_wg_tile(0, T);
  if (it < 0) return;
  AttendTile ti = attend_tile_at(a, it, QT, nchk, per);
  auto issue_next = [&]() {
    if (it < 0) return;
    const uint16_t* kh = KROW ? reinterpret_cast<const uint16_t*>(a.K) + (size_t)ti.h * a.n * D
                              : a.KSh + (size_t)ti.h * rp * D;
    attend_issue<D, DV, KROW>(sb[issued % R], kh, a.n, a.Wph + (size_t)ti.h * DV * rp, a.Wdh + (size_t)ti.h * rp,
                              ti.c0 + ic, wid, lane);
    ++issued;
    if (++ic == ti.nc) {
      ic = 0;
      it = attend_wg_tile(++ij, T);
      if (it >= 0) ti = attend_tile_at(a, it, QT, nchk, per);
    }
  };
  for (int i = 0; i < R - 1; ++i) issue_next();

  AttendTile tc = attend_tile_at(a, attend_wg_tile(0, T), QT, nchk, per);
  bf16x8 qraw[NQ][NK], qb[NQ][NK];
  attend_load_q<D, NQ>(a, tc.h, tc.qt * kAttendQueries + qoff, g, qraw);
  // the query fragments were loaded last: every chunk issued before them has landed too
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  attend_scale_q<D, NQ>(qraw, tc.qt * kAttendQueries + qoff, m, bl2e, qb);
  // scores of the first tile's unit 0; later tiles get theirs from the last step of the tile
  // before
  f32x16 scA[NQ], scB[NQ];
  bf16x8 pbA[NQ][2], pbB[NQ][2];
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    scA[s] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      scA[s] = mfma32(__builtin_bit_cast(bf16x8, sb[0].k[(2 * kk + g) * 64 + l32]), qb[s][kk], scA[s]);
  }
  int gbase = 0;  // global index of the current tile's first chunk
  bool drained = false;  // the tile before ended with every load of the wave drained
  for (int j = 0;;) {
    f32x16 y[NQ][NCT];
    float den[NQ][4];
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) y[s][ct] = f32x16{};
#pragma unroll
      for (int i = 0; i < 4; ++i) den[s][i] = 0.f;
      // the values of the (nonexistent) unit -1 get zero probabilities
#pragma unroll
      for (int e = 0; e < 8; ++e) pbA[s][0][e] = pbA[s][1][e] = (__bf16)0.f;
    }
    const int nc = tc.nc, c0 = tc.c0;
    const int jn = attend_wg_tile(j + 1, T);  // the next tile
    const AttendTile tn = attend_tile_at(a, jn < 0 ? 0 : jn, QT, nchk, per);
    const int qn0 = tn.qt * kAttendQueries + qoff;
    bf16x8 qbn[NQ][NK];
    // Chunk gc = gbase + c sits in ring slot gc % R (unit 2c in its lower half, 2c+1 in the
    // upper).  Its loads were issued R-1 chunks ahead and are waited for at the barrier of chunk
    // gc-1, with the chunks after it still in flight; that barrier also frees slot
    // (gc-1) % R, whose last reads (values of unit 2c-1) come before it.
    // The next tile's query fragments are requested two chunks before the end of this one
    // (MODE 1, after that chunk's loads) and stay in flight behind the chunk awaited at the
    // next barrier (MODE 2).  At the last chunk (MODE 3) they are scaled right after its
    // barrier, before any further load is issued, so that the wait the compiler puts in front
    // of their first use covers nothing younger than them; its second step then scores the
    // next tile's first unit (the first chunk of the next tile is resident by then) under the
    // next tile's queries.  A one-chunk tile requests and scales them after its barrier
    // (MODE 4), and the last tile of the workgroup has none to request (MODE 0 throughout).
    // A tile of at least kAttendLongTile chunks moves both tile-end costs off the chunk waits:
    //  * its next queries are requested five chunks before the end (MODE 1) and scaled after
    //    the barrier three chunks before it (MODE 5), where the compiler's wait for them also
    //    drains the chunks requested before that barrier, which were due one chunk later;
    //  * its last chunk (MODE 6) issues no load at its barrier.  At the tile end every load of
    //    the wave is drained before the output stores, and the deferred chunk is requested
    //    after them.  The first chunk of the next tile then waits for nothing (its chunk
    //    landed before the stores), so the stores complete behind a whole chunk of work
    //    instead of holding up the first count-based wait that follows them (stores and loads
    //    share the one vector-memory counter).
    auto chunk = [&](int c, auto mode_c) {
      constexpr int MODE = decltype(mode_c)::value;
      const int gc = gbase + c;
      const int bc = gc % R, bn = (gc + 1) % R, bl = c == 0 ? bc : (gc + R - 1) % R;
      const int left = lim - (c0 + c) * 64;  // rows of this chunk below the bound
      if (MASK && left < 32) attend_mask<NQ>(scA, left, g);
      attend_step<D, DV, NQ>(sb[bc], 1, sb[bc], 0, sb[bl], c == 0 ? 0 : 1, qb, y, den, scA, scB, pbA, pbB, g, l32);
      attend_pin<NQ>(pbB, den);
      // chunk gc+1 landed; the chunks issued after it (at most R-2) may still be loading, and
      // so may the next tile's query fragments once requested
      // (after a tile end that drained every load, the first chunk's is already resident)
      if (!(c == 0 && drained))
        attend_wait<D, DV, (MODE == 2 || MODE == 3 || MODE == 5) ? QN : 0>(issued - (gc + 2), wid);
      __syncthreads();
      if constexpr (MODE == 4) attend_load_q<D, NQ>(a, tn.h, qn0, g, qraw);
      if constexpr (MODE == 3 || MODE == 4 || MODE == 5) {
        attend_scale_q<D, NQ>(qraw, qn0, m, bl2e, qbn);
        attend_pin_q<D, NQ>(qbn);
      }
      if constexpr (MODE != 6) issue_next();
      if constexpr (MODE == 1) attend_load_q<D, NQ>(a, tn.h, qn0, g, qraw);
      if (MASK && left < 64) attend_mask<NQ>(scB, left - 32, g);
      if constexpr (MODE == 3 || MODE == 4 || MODE == 6)
        attend_step<D, DV, NQ>(sb[bn], 0, sb[bc], 1, sb[bc], 0, qbn, y, den, scB, scA, pbB, pbA, g, l32);
      else  // at the last chunk of the last tile the next unit's scores are never used
        attend_step<D, DV, NQ>(sb[bn], 0, sb[bc], 1, sb[bc], 0, qb, y, den, scB, scA, pbB, pbA, g, l32);
      attend_pin<NQ>(pbA, den);
    };
    if (jn < 0) {
      for (int c = 0; c < nc; ++c) chunk(c, std::integral_constant<int, 0>{});
    } else if (nc == 1) {
      chunk(0, std::integral_constant<int, 4>{});
    } else if (nc >= kAttendLongTile) {
      for (int c = 0; c < nc - 5; ++c) chunk(c, std::integral_constant<int, 0>{});
      chunk(nc - 5, std::integral_constant<int, 1>{});
      chunk(nc - 4, std::integral_constant<int, 2>{});
      chunk(nc - 3, std::integral_constant<int, 5>{});
      chunk(nc - 2, std::integral_constant<int, 0>{});
      chunk(nc - 1, std::integral_constant<int, 6>{});
    } else {
      const int cq = nc >= 3 ? nc - 3 : 0;
      for (int c = 0; c < cq; ++c) chunk(c, std::integral_constant<int, 0>{});
      chunk(cq, std::integral_constant<int, 1>{});
      if (nc >= 3) chunk(nc - 2, std::integral_constant<int, 2>{});
      chunk(nc - 1, std::integral_constant<int, 3>{});
    }
    // values of the last unit
    const AttendChunk<D, DV>& bz = sb[(gbase + nc - 1) % R];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const bf16x8 wf = __builtin_bit_cast(bf16x8, bz.w[(4 + 2 * (i & 1) + g) * DV + 32 * (i >> 1) + l32]);
#pragma unroll
      for (int s = 0; s < NQ; ++s) y[s][i >> 1] = mfma32(wf, pbA[s][i & 1], y[s][i >> 1]);
    }
    // outputs of this tile (after a MODE 6 chunk: behind a drain of every load in flight,
    // with the chunk its barrier did not request issued after them)
    const bool defer = jn >= 0 && nc >= kAttendLongTile;
    if (defer) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int h = tc.h, sp = tc.sp, q0 = tc.qt * kAttendQueries + qoff;
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      float dn = (den[s][0] + den[s][1]) + (den[s][2] + den[s][3]);
      dn += __shfl_xor(dn, 32, 64);
      const int q = q0 + 32 * s;
      if (q >= m) continue;
      if (a.nsplit == 1 && a.Yout) {
        float* Y = yout_row(a, h, q);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v) Y[ct * 32 + 8 * (v >> 2) + 4 * g + (v & 3)] = y[s][ct][v];
        if (g == 0) Y[DV] = dn;
      } else if (a.nsplit == 1) {
        if (!(dn > 0.f)) atomicOr(&a.flags[h], WC_DFLAG_DENOM);
        const float inv = 1.0f / dn;
        uint16_t* O = reinterpret_cast<uint16_t*>(a.O) + ((size_t)h * m + q) * DV;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int col = ct * 32 + 8 * v4 + 4 * g;
            uint16_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = bf16_bits((__bf16)(y[s][ct][4 * v4 + e] * inv));
            uint2 pk;
            pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
            pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
            *reinterpret_cast<uint2*>(O + col) = pk;
          }
      } else {
        float* Yp = a.Ypart + (((size_t)h * a.nsplit + sp) * m + q) * (DV + 1);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v) Yp[ct * 32 + 8 * (v >> 2) + 4 * g + (v & 3)] = y[s][ct][v];
        if (g == 0) Yp[DV] = dn;
      }
    }
    if (defer) issue_next();
    drained = defer;
    if (jn < 0) break;
    // the next tile: its queries are scaled and its first unit scored
    gbase += nc;
    tc = tn;
#pragma unroll
    for (int s = 0; s < NQ; ++s)
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) qb[s][kk] = qbn[s][kk];
    ++j;
  }
}

// Sum of the coreset-split partials: one wave per query row, lanes over the columns.
template <typename T, int DV>
__global__ void __launch_bounds__(64) attend_reduce_kernel(AttendArgs a) {
  constexpr int NCOL = DV / 64;  // value columns per lane: lane, lane + 64, ...
  const int q = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const size_t stride = (size_t)a.m * (DV + 1);
  const float* Yp = a.Ypart + ((size_t)h * a.nsplit * a.m + q) * (DV + 1);
  // one pass over the splits, in split order, for the normaliser and the lane's columns at once
  // (the loads of several splits go out together)
  float den = 0.f, y[NCOL];
#pragma unroll
  for (int j = 0; j < NCOL; ++j) y[j] = 0.f;
#pragma unroll 4
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* row = Yp + sp * stride;
    den += row[DV];
#pragma unroll
    for (int j = 0; j < NCOL; ++j) y[j] += row[lane + 64 * j];
  }
  if (a.Yout) {
    float* Y = yout_row(a, h, q);
#pragma unroll
    for (int j = 0; j < NCOL; ++j) Y[lane + 64 * j] = y[j];
    if (lane == 0) Y[DV] = den;
    return;
  }
  if (lane == 0 && !(den > 0.f)) atomicOr(&a.flags[h], WC_DFLAG_DENOM);
  const float inv = 1.0f / den;
  T* O = reinterpret_cast<T*>(a.O) + ((size_t)h * a.m + q) * DV;
#pragma unroll
  for (int j = 0; j < NCOL; ++j) st_elem<T>(O + lane + 64 * j, y[j] * inv);
}

// A few queries per head over a bf16 staged coreset (the compressed cache's decode step).  Each
// wave takes one 64-row chunk (a workgroup of 16 covers a 1024-row cache alone): lanes over the rows for the scores (the chunk's key pieces are
// 64 consecutive 16-byte units per column group) and over the value columns for
// Y = sum_j p_j W[j, :] (a 16-byte unit of W^T holds 8 permuted positions of one column, whose
// probabilities sit side by side in LDS).  The normaliser uses the fp32 W[:, dv].  The waves
// of a workgroup are summed in LDS; one workgroup per (chunk group, head, query) writes either
// O (when it covers every row in use) or an fp32 partial for the split reduction.
template <int D, int DV>
__global__ void __launch_bounds__(64 * kDecodeWaves) decode_kernel(AttendArgs a) {
  constexpr int NCOL = DV / 64;  // value columns per lane
  const int sp = blockIdx.x, h = blockIdx.y, q = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int rp = staged_rows(a), rows = a.scan_rows;
  const int ch = sp * kDecodeWaves + wid, row = ch * 64 + lane;
  const bool live = ch * 64 < rows;  // wave-uniform
  __shared__ __attribute__((aligned(16))) float s_p[kDecodeWaves][64];
  __shared__ float s_y[kDecodeWaves][DV + 1];
  // the chunk's W^T units are requested first, so that their latency overlaps the key loads
  const uint4* wt = reinterpret_cast<const uint4*>(a.Wph + (size_t)h * DV * rp) + (size_t)ch * 8 * DV;
  uint4 wv[8][NCOL];
  if (live) {
#pragma unroll
    for (int G = 0; G < 8; ++G)
#pragma unroll
      for (int i = 0; i < NCOL; ++i) wv[G][i] = wt[G * DV + lane + 64 * i];
  }
  // score as a base-2 exponent: the query is scaled by beta log2(e) and rounded to bf16, as in
  // the attention kernels
  float sc = 0.f;
  if (live) {
    const uint4* Qv = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.Q) + ((size_t)h * a.m + q) * D);
    const uint4* kc = reinterpret_cast<const uint4*>(a.KSh + (size_t)h * rp * D) + (size_t)ch * 8 * D;
    const float bl2e = a.beta_log2e;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int dg = 0; dg < D / 8; ++dg) {
      const uint4 qr = Qv[dg];
      const uint4 kv = kc[dg * 64 + lane];
      const uint32_t qw[4] = {qr.x, qr.y, qr.z, qr.w}, kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 lo = (__bf16)(__uint_as_float(qw[e] << 16) * bl2e);
        const __bf16 hi = (__bf16)(__uint_as_float(qw[e] & 0xffff0000u) * bl2e);
        const bf16x2 qq = {lo, hi};
        if (e & 1) s1 = __builtin_amdgcn_fdot2_f32_bf16(qq, __builtin_bit_cast(bf16x2, kw[e]), s1, false);
        else s0 = __builtin_amdgcn_fdot2_f32_bf16(qq, __builtin_bit_cast(bf16x2, kw[e]), s0, false);
      }
    }
    sc = s0 + s1;
  }
  const bool in = row < rows;
  const float p = in ? __builtin_amdgcn_exp2f(sc) : 0.f;
  float dn = in ? p * a.Wden[(size_t)h * rp + row] : 0.f;
  s_p[wid][perm32_a(lane)] = p;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) dn += __shfl_xor(dn, o, 64);
  __syncthreads();
  float y[NCOL];
#pragma unroll
  for (int i = 0; i < NCOL; ++i) y[i] = 0.f;
  if (live) {
#pragma unroll
    for (int G = 0; G < 8; ++G) {
      const float4 pa = *reinterpret_cast<const float4*>(&s_p[wid][8 * G]);
      const float4 pb = *reinterpret_cast<const float4*>(&s_p[wid][8 * G + 4]);
#pragma unroll
      for (int i = 0; i < NCOL; ++i) {
        const uint4 w = wv[G][i];
        float acc = y[i];
        acc = fmaf(pa.x, __uint_as_float(w.x << 16), acc);
        acc = fmaf(pa.y, __uint_as_float(w.x & 0xffff0000u), acc);
        acc = fmaf(pa.z, __uint_as_float(w.y << 16), acc);
        acc = fmaf(pa.w, __uint_as_float(w.y & 0xffff0000u), acc);
        acc = fmaf(pb.x, __uint_as_float(w.z << 16), acc);
        acc = fmaf(pb.y, __uint_as_float(w.z & 0xffff0000u), acc);
        acc = fmaf(pb.z, __uint_as_float(w.w << 16), acc);
        acc = fmaf(pb.w, __uint_as_float(w.w & 0xffff0000u), acc);
        y[i] = acc;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NCOL; ++i) s_y[wid][lane + 64 * i] = y[i];
  if (lane == 0) s_y[wid][DV] = dn;
  __syncthreads();
  if (wid != 0) return;
  float yt[NCOL];
#pragma unroll
  for (int i = 0; i < NCOL; ++i) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) t += s_y[w][lane + 64 * i];
    yt[i] = t;
  }
  float dt = 0.f;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) dt += s_y[w][DV];
  if (gridDim.x == 1) {
    if (lane == 0 && !(dt > 0.f)) atomicOr(&a.flags[h], WC_DFLAG_DENOM);
    const float inv = 1.0f / dt;
    uint16_t* O = reinterpret_cast<uint16_t*>(a.O) + ((size_t)h * a.m + q) * DV;
#pragma unroll
    for (int i = 0; i < NCOL; ++i) O[lane + 64 * i] = bf16_bits((__bf16)(yt[i] * inv));
  } else {
    float* Yp = a.Ypart + (((size_t)h * gridDim.x + sp) * a.m + q) * (DV + 1);
#pragma unroll
    for (int i = 0; i < NCOL; ++i) Yp[lane + 64 * i] = yt[i];
    if (lane == 0) Yp[DV] = dt;
  }
}

// Workgroups of the persistent attention kernel: the compute units of the current device (one
// workgroup each, its LDS ring takes most of a unit's LDS).
static int attend_workgroups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  return cus;
}

template <typename T, int D, int DV>
static hipError_t run_attend_core(const AttendArgs& a, hipStream_t st);

template <typename T, int D, int DV>
static hipError_t run_attend(const AttendArgs& a, hipStream_t st) {
  const int rp = staged_rows(a);
  hipLaunchKernelGGL((attend_prep_kernel<T, D, DV>), dim3(rp, a.H), dim3(128), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.m == 0) return e;
  return run_attend_core<T, D, DV>(a, st);
}

template <typename T, int D, int DV>
static hipError_t run_attend_prep(const AttendArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((attend_prep_kernel<T, D, DV>), dim3(staged_rows(a), a.H), dim3(128), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D, int DV>
static hipError_t run_attend_append(const AttendArgs& a, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL((attend_append_kernel<T, D, DV>), dim3(a.n, a.H), dim3(128), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D, int DV>
static hipError_t run_attend_all_keys(const AttendArgs& a0, hipStream_t st) {
  // bf16 keys are read by the attention in place (row-major), so only the weights are staged
  AttendArgs a = a0;
  if constexpr (sizeof(T) == 2) a.KSh = nullptr;
  const int rp = staged_rows(a);
  hipLaunchKernelGGL((attend_prep_keys_kernel<T, D, DV>), dim3(rp / 64, a.H), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.m == 0) return e;
  return run_attend_core<T, D, DV>(a, st);
}

template <typename T, int D, int DV>
static hipError_t run_attend_core(const AttendArgs& a, hipStream_t st) {
  hipError_t e;
  if constexpr (sizeof(T) == 2) {
    // persistent: one workgroup per compute unit (never more than the tiles)
    const long tiles = (long)((a.m + kAttendQueries - 1) / kAttendQueries) * a.H * a.nsplit;
    const dim3 grid((unsigned)(tiles < attend_workgroups() ? tiles : attend_workgroups()));
    if (!a.KSh)   // the all-keys pass over bf16 keys (no scan bound)
      hipLaunchKernelGGL((attend_bf16_kernel<D, DV, false, true>), grid, dim3(64 * kAttendWaves), 0, st, a);
    else if (a.scan_rows % 128 != 0)
      hipLaunchKernelGGL((attend_bf16_kernel<D, DV, true, false>), grid, dim3(64 * kAttendWaves), 0, st, a);
    else
      hipLaunchKernelGGL((attend_bf16_kernel<D, DV, false, false>), grid, dim3(64 * kAttendWaves), 0, st, a);
  } else
    hipLaunchKernelGGL((attend_kernel<T, D, DV>), dim3((a.m + 127) / 128, a.H, a.nsplit), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.nsplit > 1) {
    hipLaunchKernelGGL((attend_reduce_kernel<T, DV>), dim3(a.m, a.H), dim3(64), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  if (a.bf16) {
    if (a.d == 64) return a.dv == 64 ? run_attend<uint16_t, 64, 64>(a, st) : run_attend<uint16_t, 64, 128>(a, st);
    return a.dv == 64 ? run_attend<uint16_t, 128, 64>(a, st) : run_attend<uint16_t, 128, 128>(a, st);
  }
  if (a.d == 64) return a.dv == 64 ? run_attend<float, 64, 64>(a, st) : run_attend<float, 64, 128>(a, st);
  return a.dv == 64 ? run_attend<float, 128, 64>(a, st) : run_attend<float, 128, 128>(a, st);
}

#define WC_ATTEND_DISPATCH(FN)                                                                \
  if (a.bf16) {                                                                               \
    if (a.d == 64) return a.dv == 64 ? FN<uint16_t, 64, 64>(a, st) : FN<uint16_t, 64, 128>(a, st); \
    return a.dv == 64 ? FN<uint16_t, 128, 64>(a, st) : FN<uint16_t, 128, 128>(a, st);         \
  }                                                                                           \
  if (a.d == 64) return a.dv == 64 ? FN<float, 64, 64>(a, st) : FN<float, 64, 128>(a, st);     \
  return a.dv == 64 ? FN<float, 128, 64>(a, st) : FN<float, 128, 128>(a, st);

hipError_t launch_attend_prep(const AttendArgs& a, hipStream_t st) { WC_ATTEND_DISPATCH(run_attend_prep) }
hipError_t launch_attend_append(const AttendArgs& a, hipStream_t st) { WC_ATTEND_DISPATCH(run_attend_append) }
hipError_t launch_attend_core(const AttendArgs& a, hipStream_t st) {
  if (a.m == 0) return hipSuccess;
  WC_ATTEND_DISPATCH(run_attend_core)
}

template <typename T, int D, int DV>
static hipError_t run_decode(const AttendArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) != 2) {
    return hipErrorInvalidValue;
  } else {
    const int ns = decode_splits(a.scan_rows);
    hipLaunchKernelGGL((decode_kernel<D, DV>), dim3(ns, a.H, a.m), dim3(64 * kDecodeWaves), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    AttendArgs r = a;
    r.nsplit = ns;
    r.Yout = nullptr;
    hipLaunchKernelGGL((attend_reduce_kernel<T, DV>), dim3(a.m, a.H), dim3(64), 0, st, r);
    return hipGetLastError();
  }
}

hipError_t launch_decode(const AttendArgs& a, hipStream_t st) {
  if (a.m == 0) return hipSuccess;
  if (!a.bf16 || a.m > kDecodeMaxQueries || a.scan_rows < 1 || a.scan_rows > staged_rows(a) || !a.Q || !a.O ||
      (decode_splits(a.scan_rows) > 1 && !a.Ypart))
    return hipErrorInvalidValue;
  WC_ATTEND_DISPATCH(run_decode)
}

hipError_t launch_attend_all_keys(const AttendArgs& a, hipStream_t st) {
  if (a.bf16) {
    if (a.d == 64)
      return a.dv == 64 ? run_attend_all_keys<uint16_t, 64, 64>(a, st) : run_attend_all_keys<uint16_t, 64, 128>(a, st);
    return a.dv == 64 ? run_attend_all_keys<uint16_t, 128, 64>(a, st) : run_attend_all_keys<uint16_t, 128, 128>(a, st);
  }
  if (a.d == 64) return a.dv == 64 ? run_attend_all_keys<float, 64, 64>(a, st) : run_attend_all_keys<float, 64, 128>(a, st);
  return a.dv == 64 ? run_attend_all_keys<float, 128, 64>(a, st) : run_attend_all_keys<float, 128, 128>(a, st);
}

}  // namespace wc
