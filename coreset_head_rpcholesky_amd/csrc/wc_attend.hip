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
//   normaliser Y[:, dv] is an fp32 dot product of P with W[:, dv] on the vector units.
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

template <typename T, int D, int DV>
__global__ void __launch_bounds__(128) attend_prep_kernel(AttendArgs a) {
  constexpr bool SPLIT = sizeof(T) == 4;
  const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int rp = (a.r + 63) & ~63;
  const int rk = a.rank[h];
  const bool valid = j < rk;
  const int s = valid ? a.pivots[(size_t)h * a.r + j] : 0;
  const T* K = reinterpret_cast<const T*>(a.K) + ((size_t)h * a.n + s) * D;
  for (int e = tid; e < D; e += 128) {
    const float v = valid ? ld_elem<T>(K + e) : 0.f;
    __bf16 hi, lo;
    split_bf16(v, hi, lo);
    a.KSh[((size_t)h * rp + j) * D + e] = bf16_bits(hi);
    if (SPLIT) a.KSl[((size_t)h * rp + j) * D + e] = bf16_bits(lo);
  }
  const int p = perm32_a(j);
  const float* W = a.W + ((size_t)h * a.r + (valid ? j : 0)) * (DV + 1);
  for (int c = tid; c < DV; c += 128) {
    const float w = valid ? W[c] : 0.f;
    __bf16 hi, lo;
    split_bf16(w, hi, lo);
    a.Wph[((size_t)h * DV + c) * rp + p] = bf16_bits(hi);
    if (SPLIT) a.Wpl[((size_t)h * DV + c) * rp + p] = bf16_bits(lo);
  }
  if (tid == 0) a.Wden[(size_t)h * rp + j] = valid ? W[DV] : 0.f;
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
  const int m = a.m, rp = (a.r + 63) & ~63, nchk = rp / 32;
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
      const size_t src = (size_t)(c * 32 + jj) * D + 8 * k8;
      *reinterpret_cast<uint4*>(sKh + jj * KP + 8 * k8) = *reinterpret_cast<const uint4*>(KSh + src);
      if (SPLIT) *reinterpret_cast<uint4*>(sKl + jj * KP + 8 * k8) = *reinterpret_cast<const uint4*>(KSl + src);
    }
    for (int e = tid; e < DV * 4; e += 256) {
      const int cc = e / 4, k8 = e % 4;
      const size_t src = (size_t)cc * rp + c * 32 + 8 * k8;
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
      const float p = __builtin_amdgcn_exp2f(sc[v] * bl2e);
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
  if (a.nsplit == 1) {
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

// bf16 inputs: each wave takes NQ x 32 queries; coreset chunks of 64 are double-buffered in
// LDS and the next chunk is loaded into registers while the current one is computed; one
// barrier per chunk.
template <int D, int DV, int NQ>
__global__ void __launch_bounds__(256) attend_bf16_kernel(AttendArgs a) {
  constexpr int CH = 64, KP = D + 8, WP = CH + 8, NCT = DV / 32;
  constexpr int QPB = 4 * 32 * NQ;  // queries per workgroup
  constexpr int KV = CH * D / 8 / 256;   // uint4 of K_S per thread per chunk
  constexpr int WV = DV * CH / 8 / 256;  // uint4 of W^T per thread per chunk
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][CH * KP];
  __shared__ __attribute__((aligned(16))) __bf16 sW[2][DV * WP];
  __shared__ float sWd[2][CH];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y, sp = blockIdx.z;
  const int m = a.m, rp = (a.r + 63) & ~63, nchk = rp / CH;
  const float bl2e = a.beta_log2e;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.Q) + (size_t)h * m * D;
  const int qbase = blockIdx.x * QPB + wid * 32 * NQ;

  bf16x8 qb[NQ][D / 16];
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    const int q = qbase + 32 * s + l32;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (q < m) {
        qb[s][kk] = *reinterpret_cast<const bf16x8*>(Q + (size_t)q * D + 16 * kk + 8 * g);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[s][kk][e] = (__bf16)0.f;
      }
    }
  }
  f32x16 y[NQ][NCT];
#pragma unroll
  for (int s = 0; s < NQ; ++s)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) y[s][ct][v] = 0.f;
  float den[NQ];
#pragma unroll
  for (int s = 0; s < NQ; ++s) den[s] = 0.f;
  const int per = (nchk + a.nsplit - 1) / a.nsplit;
  const int cb = sp * per, ce = min(nchk, cb + per);
  const uint16_t* KSh = a.KSh + (size_t)h * rp * D;
  const uint16_t* Wph = a.Wph + (size_t)h * DV * rp;
  const float* Wden = a.Wden + (size_t)h * rp;
  uint4 kreg[KV], wreg[WV];
  float dreg = 0.f;
  auto fetch = [&](int c) {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int e = tid + 256 * i, jj = e / (D / 8), k8 = e % (D / 8);
      kreg[i] = *reinterpret_cast<const uint4*>(KSh + (size_t)(c * CH + jj) * D + 8 * k8);
    }
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int e = tid + 256 * i, cc = e / (CH / 8), k8 = e % (CH / 8);
      wreg[i] = *reinterpret_cast<const uint4*>(Wph + (size_t)cc * rp + c * CH + 8 * k8);
    }
    if (tid < CH) dreg = Wden[c * CH + tid];
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int e = tid + 256 * i, jj = e / (D / 8), k8 = e % (D / 8);
      *reinterpret_cast<uint4*>(&sK[buf][jj * KP + 8 * k8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int e = tid + 256 * i, cc = e / (CH / 8), k8 = e % (CH / 8);
      *reinterpret_cast<uint4*>(&sW[buf][cc * WP + 8 * k8]) = wreg[i];
    }
    if (tid < CH) sWd[buf][tid] = dreg;
  };
  if (cb < ce) {
    fetch(cb);
    store(0);
  }
  for (int c = cb; c < ce; ++c) {
    const int buf = (c - cb) & 1;
    __syncthreads();
    // both sub-chunks' score MFMAs are issued first, so the exponentials of one overlap the
    // matrix-core work of the other
    constexpr int NSUB = CH / 32;
    f32x16 sc[NSUB][NQ];
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
      for (int s = 0; s < NQ; ++s)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[sub][s][v] = 0.f;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 kh = *reinterpret_cast<const bf16x8*>(&sK[buf][(sub * 32 + l32) * KP + 16 * kk + 8 * g]);
#pragma unroll
        for (int s = 0; s < NQ; ++s) sc[sub][s] = mfma32(kh, qb[s][kk], sc[sub][s]);
      }
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      bf16x8 pb[NQ][2];
#pragma unroll
      for (int s = 0; s < NQ; ++s)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(sc[sub][s][v] * bl2e);
          den[s] = fmaf(p, sWd[buf][sub * 32 + 8 * (v >> 2) + 4 * g + (v & 3)], den[s]);
          pb[s][v >> 3][v & 7] = (__bf16)p;
        }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const bf16x8 wh = *reinterpret_cast<const bf16x8*>(&sW[buf][(ct * 32 + l32) * WP + sub * 32 + 16 * qq + 8 * g]);
#pragma unroll
          for (int s = 0; s < NQ; ++s) y[s][ct] = mfma32(wh, pb[s][qq], y[s][ct]);
        }
    }
    if (c + 1 < ce) {  // the other buffer was last read before this iteration's barrier
      fetch(c + 1);
      store(buf ^ 1);
    }
  }
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    const float dn = den[s] + __shfl_xor(den[s], 32, 64);
    const int q = qbase + 32 * s + l32;
    if (q >= m) continue;
    if (a.nsplit == 1) {
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
}

template <typename T, int DV>
__global__ void __launch_bounds__(256) attend_reduce_kernel(AttendArgs a) {
  const int h = blockIdx.y;
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= a.m) return;
  const size_t stride = (size_t)a.m * (DV + 1);
  const float* Yp = a.Ypart + ((size_t)h * a.nsplit * a.m + q) * (DV + 1);
  float den = 0.f;
  for (int sp = 0; sp < a.nsplit; ++sp) den += Yp[sp * stride + DV];
  if (!(den > 0.f)) atomicOr(&a.flags[h], WC_DFLAG_DENOM);
  const float inv = 1.0f / den;
  T* O = reinterpret_cast<T*>(a.O) + ((size_t)h * a.m + q) * DV;
  for (int c = 0; c < DV; ++c) {
    float y = 0.f;
    for (int sp = 0; sp < a.nsplit; ++sp) y += Yp[sp * stride + c];
    st_elem<T>(O + c, y * inv);
  }
}

template <typename T, int D, int DV>
static hipError_t run_attend(const AttendArgs& a, hipStream_t st) {
  static_assert(kAttendNQ == 1 || kAttendNQ == 2, "32 or 64 queries per wave");
  const int rp = (a.r + 63) & ~63;
  hipLaunchKernelGGL((attend_prep_kernel<T, D, DV>), dim3(rp, a.H), dim3(128), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.m == 0) return e;
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((attend_bf16_kernel<D, DV, kAttendNQ>), dim3((a.m + 128 * kAttendNQ - 1) / (128 * kAttendNQ), a.H, a.nsplit), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attend_kernel<T, D, DV>), dim3((a.m + 127) / 128, a.H, a.nsplit), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.nsplit > 1) {
    hipLaunchKernelGGL((attend_reduce_kernel<T, DV>), dim3((a.m + 255) / 256, a.H), dim3(256), 0, st, a);
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

}  // namespace wc
