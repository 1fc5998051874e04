// Rotate-then-pool block summaries (Geometry Matters in Packed 3D Attention,
// project page Ch. 3 "Rotate first, then pool"; paper summary §3.2, §B.5).
//
// One workgroup per (block, batch). Members are visited in canonical
// within-block-slot order, so the fp32 sums -- and hence the summaries -- are
// the same bits under any packing of the tokens. Threads own channel pairs of
// the token's contiguous [H, D] row, so each member read is one coalesced
// run of H*D elements. HBM-bound: every K and V element is read once.
#include "launch.hpp"

namespace pk {

constexpr int kMaxVol = 512;  // members staged in LDS per pass

template <typename T>
__global__ void k_summarize(Geo g, const void *geom, const T *k, const T *v, T *ks, T *vs) {
  __shared__ int s_slot[kMaxVol];
  __shared__ int s_count;
  const int m = blockIdx.x, b = blockIdx.y;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int oz = (m / (g.My * g.Mx)) * g.bz, oy = ((m / g.Mx) % g.My) * g.by,
            ox = (m % g.Mx) * g.bx;
  const int half = g.D / 2, da = g.D / 3, npair = g.H * half;
  // Each thread keeps up to 2 channel pairs (npair <= 2 * blockDim.x).
  float ka[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, va[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  if (threadIdx.x == 0) s_count = 0;
  for (int r0 = 0; r0 < g.vol; r0 += kMaxVol) {
    int nr = min(kMaxVol, g.vol - r0);
    __syncthreads();
    for (int r = threadIdx.x; r < nr; r += blockDim.x) {
      int rr = r0 + r;
      int z = oz + rr / (g.by * g.bx), y = oy + (rr / g.bx) % g.by, x = ox + rr % g.bx;
      int j = -1;
      if (z < g.Z && y < g.Y && x < g.X) j = slot[site_of(g, z, y, x)];
      s_slot[r] = j;
      if (j >= 0) atomicAdd(&s_count, 1);
    }
    __syncthreads();
    for (int r = 0; r < nr; r++) {
      int j = s_slot[r];
      if (j < 0) continue;
      int rr = r0 + r;
      int c3[3] = {oz + rr / (g.by * g.bx), oy + (rr / g.bx) % g.by, ox + rr % g.bx};
      const int64_t row = ((int64_t)b * g.N + j) * g.H * g.D;
#pragma unroll
      for (int u = 0; u < 2; u++) {
        int t = threadIdx.x + u * blockDim.x;
        if (t < npair) {
          int h = t / half, d0 = 2 * (t % half);
          int a = d0 / da, p = (d0 % da) / 2;
          const T *kp = k + row + h * g.D + d0;
          const T *vp = v + row + h * g.D + d0;
          float k0 = to_f32(kp[0]), k1 = to_f32(kp[1]);
          rotate(k0, k1, rope_cs(tab, g, a, c3[a], p));
          ka[u][0] += k0;
          ka[u][1] += k1;
          va[u][0] += to_f32(vp[0]);
          va[u][1] += to_f32(vp[1]);
        }
      }
    }
  }
  __syncthreads();
  const int cnt = s_count;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    int t = threadIdx.x + u * blockDim.x;
    if (t < npair) {
      int h = t / half, d0 = 2 * (t % half);
      int64_t o = (((int64_t)b * g.H + h) * g.M + m) * g.D + d0;
      // mean = sum / count (division, as written in the definition)
      ks[o] = from_f32<T>(cnt > 0 ? ka[u][0] / (float)cnt : 0.0f);
      ks[o + 1] = from_f32<T>(cnt > 0 ? ka[u][1] / (float)cnt : 0.0f);
      vs[o] = from_f32<T>(cnt > 0 ? va[u][0] / (float)cnt : 0.0f);
      vs[o + 1] = from_f32<T>(cnt > 0 ? va[u][1] / (float)cnt : 0.0f);
    }
  }
}

hipError_t launch_summarize(const Geo &g, int dtype, const void *geom, const void *k,
                            const void *v, void *ks, void *vs, hipStream_t s) {
  int npair = g.H * g.D / 2;
  int threads = npair <= 256 ? ((npair + 63) / 64) * 64 : 256;
  if (npair > 2 * threads) return hipErrorInvalidValue;  // host checks H*D <= 1024
  dim3 grid((unsigned)g.M, (unsigned)g.B);
  if (dtype == PACK3D_BF16)
    hipLaunchKernelGGL(k_summarize<bf16>, grid, dim3(threads), 0, s, g, geom,
                       static_cast<const bf16 *>(k), static_cast<const bf16 *>(v),
                       static_cast<bf16 *>(ks), static_cast<bf16 *>(vs));
  else
    hipLaunchKernelGGL(k_summarize<float>, grid, dim3(threads), 0, s, g, geom,
                       static_cast<const float *>(k), static_cast<const float *>(v),
                       static_cast<float *>(ks), static_cast<float *>(vs));
  return hipGetLastError();
}

}  // namespace pk
