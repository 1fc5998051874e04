// Tokenwise gated mix of the two branches (Geometry Matters in Packed 3D
// Attention, paper summary §3.3): g = sigmoid(G), O = (1-g) O_loc + g O_glob.
#include "launch.hpp"

namespace pk {

template <typename T>
__global__ void k_mix(int64_t rows, int D, const T *gate, const T *ol, const T *og, T *o) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * D) return;
  int64_t row = t / D;
  float gl = to_f32(gate[row]);
  float gg = 1.0f / (1.0f + expf(-gl));
  float r = (1.0f - gg) * to_f32(ol[t]) + gg * to_f32(og[t]);
  o[t] = from_f32<T>(r);
}

hipError_t launch_mix(const Geo &g, int dtype, const void *gate, const void *ol, const void *og,
                      void *o, hipStream_t s) {
  int64_t rows = (int64_t)g.B * g.N * g.H;
  dim3 grid((unsigned)((rows * g.D + 255) / 256));
  if (dtype == PACK3D_BF16)
    hipLaunchKernelGGL(k_mix<bf16>, grid, dim3(256), 0, s, rows, g.D,
                       static_cast<const bf16 *>(gate), static_cast<const bf16 *>(ol),
                       static_cast<const bf16 *>(og), static_cast<bf16 *>(o));
  else
    hipLaunchKernelGGL(k_mix<float>, grid, dim3(256), 0, s, rows, g.D,
                       static_cast<const float *>(gate), static_cast<const float *>(ol),
                       static_cast<const float *>(og), static_cast<float *>(o));
  return hipGetLastError();
}

}  // namespace pk
