// Key centring (gist.science/de/paper/2602.10056, "Methodik" part 3: softmax attention is
// invariant under a global shift of the keys, which are re-centred by their mean):
//     Kc = K - mean of the head's keys,
// formed in fp64 and stored in the input precision (fp32 round to nearest; bf16 through fp32,
// round to nearest even).  The mean is a fixed-order fp64 sum: per 1024-row block, then over
// the blocks.
#include "wc_device.h"
#include "wc_kernels.h"

namespace wc {

namespace {

// Block sums: thread t adds column t % d over rows t / d, t / d + 256 / d, ... of the block;
// the 256 / d row lanes of a column are then added in order.
template <typename T>
__global__ void __launch_bounds__(256) center_part_kernel(CenterArgs a) {
  __shared__ double red[256];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lanes = 256 / a.d, e = tid % a.d, lr = tid / a.d;
  const T* K = reinterpret_cast<const T*>(a.K) + (size_t)h * a.n * a.d;
  double s = 0.0;
  const int i1 = min(a.n, (b + 1) * kCenterRows);
  for (int i = b * kCenterRows + lr; i < i1; i += lanes) s += (double)ld_elem<T>(K + (size_t)i * a.d + e);
  red[tid] = s;
  __syncthreads();
  if (tid < a.d) {
    double t = 0.0;
    for (int l = 0; l < lanes; ++l) t += red[l * a.d + tid];
    a.part[((size_t)h * a.nblk + b) * a.d + tid] = t;
  }
}

__global__ void __launch_bounds__(128) center_mean_kernel(CenterArgs a) {
  const int h = blockIdx.x, e = threadIdx.x;
  if (e >= a.d) return;
  double t = 0.0;
  for (int b = 0; b < a.nblk; ++b) t += a.part[((size_t)h * a.nblk + b) * a.d + e];
  a.mean[(size_t)h * a.d + e] = t / (double)a.n;
}

template <typename T>
__global__ void __launch_bounds__(256) center_sub_kernel(CenterArgs a) {
  const int h = blockIdx.y;
  const size_t total = (size_t)a.n * a.d;
  const T* K = reinterpret_cast<const T*>(a.K) + (size_t)h * total;
  T* Kc = reinterpret_cast<T*>(a.Kc) + (size_t)h * total;
  const double* mean = a.mean + (size_t)h * a.d;
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < total; x += (size_t)gridDim.x * 256) {
    const float v = (float)((double)ld_elem<T>(K + x) - mean[x % a.d]);
    st_elem<T>(Kc + x, v);
  }
}

template <typename T>
hipError_t run_center(const CenterArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((center_part_kernel<T>), dim3(a.nblk, a.H), dim3(256), 0, st, a);
  hipLaunchKernelGGL(center_mean_kernel, dim3(a.H), dim3(128), 0, st, a);
  const size_t total = (size_t)a.n * a.d;
  const size_t blocks = (total + 255) / 256;
  const int gx = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL((center_sub_kernel<T>), dim3(gx, a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_center(const CenterArgs& a, hipStream_t st) {
  return a.bf16 ? run_center<uint16_t>(a, st) : run_center<float>(a, st);
}

}  // namespace wc
