// Materialised axial RoPE at grid coordinates (Geometry Matters in Packed 3D
// Attention, project page Ch. 3, Contract 3; paper summary §B.2): every
// channel pair of axis chunk a turns by c_a * base^(-2p/(D/3)).
#include "launch.hpp"

namespace pk {

template <typename T>
__global__ void k_rope(Geo g, const int32_t *coords, const T *x, T *y) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one channel pair
  int64_t pairs = (int64_t)g.B * g.N * g.H * (g.D / 2);
  if (t >= pairs) return;
  int half = g.D / 2, da = g.D / 3;
  int pp = (int)(t % half);
  int64_t row = t / half;
  int i = (int)((row / g.H) % g.N);
  int d0 = 2 * pp, a = d0 / da, p = (d0 % da) / 2;
  int c = coords[3 * (int64_t)i + a];
  float2 cs = rope_cs_direct(g.rope_base, g.D, c, p);
  float x0 = to_f32(x[row * g.D + d0]), x1 = to_f32(x[row * g.D + d0 + 1]);
  rotate(x0, x1, cs);
  y[row * g.D + d0] = from_f32<T>(x0);
  y[row * g.D + d0 + 1] = from_f32<T>(x1);
}

hipError_t launch_rope(const Geo &g, int dtype, const int32_t *coords, const void *x, void *y,
                       hipStream_t s) {
  int64_t pairs = (int64_t)g.B * g.N * g.H * (g.D / 2);
  dim3 grid((unsigned)((pairs + 255) / 256));
  if (dtype == PACK3D_BF16)
    hipLaunchKernelGGL(k_rope<bf16>, grid, dim3(256), 0, s, g, coords,
                       static_cast<const bf16 *>(x), static_cast<bf16 *>(y));
  else
    hipLaunchKernelGGL(k_rope<float>, grid, dim3(256), 0, s, g, coords,
                       static_cast<const float *>(x), static_cast<float *>(y));
  return hipGetLastError();
}

}  // namespace pk
