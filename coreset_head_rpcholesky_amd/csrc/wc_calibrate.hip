// Calibration kernels for the rooflines.  They measure the rates this GPU attains on the
// operations that bound the hot path's kernels, so that the datasheet peaks the rooflines are
// quoted against (HBM 8 TB/s, bf16 matrix cores 2.5 PFLOP/s, fp32 matrix cores 157.3 TFLOP/s)
// can be reported with what the part actually sustains beside them.  None of this is a step of
// the method:
//   WC_CAL_READ       a stream of 16-byte nontemporal loads over a buffer, sixteen in flight per
//                     lane on 8192 workgroups (the pivot step's factor stream is such a read;
//                     of the shapes tried, 4 to 16 loads per lane on 2048 to 16384 workgroups,
//                     with and without the nontemporal hint, this one streamed fastest);
//   WC_CAL_COPY       16-byte nontemporal loads and stores of one buffer into another, eight
//                     of each in flight per lane;
//   WC_CAL_MFMA_BF16  chains of v_mfma_f32_32x32x16_bf16 (the attention's instruction) on
//                     register operands: two waves per SIMD, eight independent accumulators
//                     per wave, nothing else in the loop;
//   WC_CAL_MFMA_F32   the same with v_mfma_f32_32x32x2_f32 (the fp32 factor products of the
//                     block selection and the union weights).
// The matrix-core kernels read the shader clock (s_memtime) and the 100 MHz reference clock
// (s_memrealtime) at the start and end of workgroup 0, so the clock the part holds under that
// load follows from the two differences.
#include <hip/hip_runtime.h>

#include "../../include/wc.h"
#include "wc_device.h"

namespace wc {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCalThreads = 256;
constexpr int kCalStreamGroups = 8192;  // 32 workgroups per compute unit
constexpr int kCalReadUnroll = 16, kCalCopyUnroll = 8;  // 16-byte loads in flight per lane
constexpr int kCalMfmaGroups = 512;     // 4 waves each: two waves per SIMD on 256 CUs
constexpr int kCalAcc = 8;              // independent accumulators per wave

__device__ __forceinline__ uint32_t wave_xor(uint32_t x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  return x;
}

// Every lane XORs the 16-byte words it reads, so that no load is dead; one word per wave out.
__global__ void __launch_bounds__(kCalThreads) cal_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                               uint32_t* __restrict__ out) {
  constexpr int U = kCalReadUnroll;
  const size_t stride = (size_t)gridDim.x * kCalThreads;
  size_t i = (size_t)blockIdx.x * kCalThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t x = wave_xor(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kCalThreads / 64) + (threadIdx.x >> 6)] = x;
}

__global__ void __launch_bounds__(kCalThreads) cal_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                               size_t n16) {
  constexpr int U = kCalCopyUnroll;
  const size_t stride = (size_t)gridDim.x * kCalThreads;
  size_t i = (size_t)blockIdx.x * kCalThreads + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Clock readings of workgroup 0 (shader clock, reference clock) at the start and the end.
__device__ __forceinline__ void cal_clock(uint64_t* clocks, int slot) {
  if (clocks && blockIdx.x == 0 && threadIdx.x == 0) {
    const uint64_t c = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    clocks[2 * slot] = c;
    clocks[2 * slot + 1] = r;
  }
}

// All operands are 1, so every MFMA adds K (16) to each accumulator element; out[wave] is lane
// 0's sum over its accumulators' elements, 8 * 16 * 16 * iters, exact while that stays below
// 2^24.
__global__ void __launch_bounds__(kCalThreads, 2) cal_mfma_bf16_kernel(int iters, float* __restrict__ out,
                                                                      uint64_t* clocks) {
  cal_clock(clocks, 0);
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)1.0f;
  f32x16 acc[kCalAcc];
#pragma unroll
  for (int k = 0; k < kCalAcc; ++k) acc[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kCalAcc; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kCalAcc; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[k][v];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kCalThreads / 64) + (threadIdx.x >> 6)] = s;
  __syncthreads();
  cal_clock(clocks, 1);
}

// As above with v_mfma_f32_32x32x2_f32: each MFMA adds 2 to every element, out[wave] =
// 8 * 16 * 2 * iters.
__global__ void __launch_bounds__(kCalThreads, 2) cal_mfma_f32_kernel(int iters, float* __restrict__ out,
                                                                     uint64_t* clocks) {
  cal_clock(clocks, 0);
  f32x16 acc[kCalAcc];
#pragma unroll
  for (int k = 0; k < kCalAcc; ++k) acc[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kCalAcc; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(1.0f, 1.0f, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kCalAcc; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[k][v];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kCalThreads / 64) + (threadIdx.x >> 6)] = s;
  __syncthreads();
  cal_clock(clocks, 1);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace
}  // namespace wc

extern "C" {

wc_status wc_calibrate(int32_t kind, const void* src, void* dst, size_t bytes, int32_t iters, uint64_t* clocks,
                       void* stream) {
  using namespace wc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!dst || !aligned16(dst) || ((uintptr_t)clocks & 7u) != 0) return WC_ERR_INVALID_ARG;
  if (kind == WC_CAL_READ || kind == WC_CAL_COPY) {
    if (!src || !aligned16(src) || bytes == 0 || bytes % 16 != 0) return WC_ERR_INVALID_ARG;
    const char* s = static_cast<const char*>(src);
    char* d = static_cast<char*>(dst);
    if (kind == WC_CAL_COPY && s < d + bytes && d < s + bytes) return WC_ERR_INVALID_ARG;
    if (kind == WC_CAL_READ)
      hipLaunchKernelGGL(cal_read_kernel, dim3(kCalStreamGroups), dim3(kCalThreads), 0, st,
                         static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(dst));
    else
      hipLaunchKernelGGL(cal_copy_kernel, dim3(kCalStreamGroups), dim3(kCalThreads), 0, st,
                         static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  } else if (kind == WC_CAL_MFMA_BF16 || kind == WC_CAL_MFMA_F32) {
    if (iters < 1) return WC_ERR_INVALID_ARG;
    if (kind == WC_CAL_MFMA_BF16)
      hipLaunchKernelGGL(cal_mfma_bf16_kernel, dim3(kCalMfmaGroups), dim3(kCalThreads), 0, st, (int)iters,
                         static_cast<float*>(dst), clocks);
    else
      hipLaunchKernelGGL(cal_mfma_f32_kernel, dim3(kCalMfmaGroups), dim3(kCalThreads), 0, st, (int)iters,
                         static_cast<float*>(dst), clocks);
  } else {
    return WC_ERR_INVALID_ARG;
  }
  return hipGetLastError() == hipSuccess ? WC_OK : WC_ERR_DEVICE;
}

}  // extern "C"
