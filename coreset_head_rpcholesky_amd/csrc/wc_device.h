// Device-side helpers shared by the WildCat HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace wc {

// fn(std::integral_constant<int, I>{}) for I = I0 .. N-1: loop bodies specialised per step.
template <int I, int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>{});
    static_for<I + 1, N>(fn);
  }
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Debug builds (WC_DEBUG=1) check every index that a kernel reads from device memory before
// dereferencing it: the pivot indices handed in by the caller, which the host cannot see.  An
// index outside [0, n) is not used (the slot counts as empty) and flag bit 16 (WC_FLAG_BOUNDS)
// is OR-ed into the head's flags when the kernel has them; the checks report instead of
// trapping, so the device stays usable and the flags name the head.  Other builds trust the
// ranges the entry points document.
#ifndef WC_DEBUG
#define WC_DEBUG 0
#endif
__device__ __forceinline__ bool wc_index_ok(int i, int n, uint32_t* flag) {
  if constexpr (WC_DEBUG == 0) {
    return true;
  } else {
    const bool ok = i >= 0 && i < n;
    if (!ok && flag) atomicOr(flag, 16u);  // WC_DFLAG_BOUNDS
    return ok;
  }
}

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---- bf16 <-> f32 ---------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }

// hi + lo split of an fp32 value into two bf16 parts: x ~= hi + lo to ~16 mantissa bits.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// Input element loads: T is float or uint16_t (bf16 bits).
template <typename T> __device__ __forceinline__ float ld_elem(const T* p);
template <> __device__ __forceinline__ float ld_elem<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p) {
  return bf16_bits_to_f32(*p);
}
template <typename T> __device__ __forceinline__ void st_elem(T* p, float v);
template <> __device__ __forceinline__ void st_elem<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st_elem<uint16_t>(uint16_t* p, float v) {
  __bf16 b = (__bf16)v;
  *p = __builtin_bit_cast(uint16_t, b);
}

// ---- MFMA -------------------------------------------------------------------------------
// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane l (g = l / 32): A holds A[l % 32][8g .. 8g+7], B holds B[8g .. 8g+7][l % 32];
// accumulator register v holds D[8*(v/4) + 4g + v%4][l % 32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- Philox4x64-10 (Salmon et al., SC'11) ---------------------------------------------------
// Pivot step t of head h draws u = (x0 >> 40) * 2^-24 from the block with counter
// (t, h, 0, 0) and key (seed, 0).
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint32_t head, uint32_t step) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = step, x1 = head, x2 = 0, x3 = 0, k0 = seed, k1 = 0;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) { k0 += W0; k1 += W1; }
    const uint64_t hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
    const uint64_t hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
  }
  return (float)(x0 >> 40) * 0x1p-24f;
}

__device__ __forceinline__ float pivot_uniform(const float* u_forced, uint64_t seed, int head,
                                               int r, int step) {
  return u_forced ? u_forced[(size_t)head * r + step] : philox_uniform(seed, head, step);
}

// ---- wave-level fp64 scans and reductions (deterministic order) --------------------------
__device__ __forceinline__ double shfl_up_d(double x, int delta) { return __shfl_up(x, delta, kWave); }
__device__ __forceinline__ double shfl_xor_d(double x, int m) { return __shfl_xor(x, m, kWave); }

// Inclusive scan across the 64 lanes (Hillis-Steele, fixed order).
__device__ __forceinline__ double wave_incl_scan(double x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = shfl_up_d(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Sum across the 64 lanes, identical result in every lane.
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += shfl_xor_d(x, m);
  return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

// Probability mass of a residual: max(diag, 0), with NaN kept so that it poisons the total.
__device__ __forceinline__ double mass_of(float dg) {
  return (dg > 0.f || dg != dg) ? (double)dg : 0.0;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

}  // namespace wc
