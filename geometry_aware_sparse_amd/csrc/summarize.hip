// Rotate-then-pool block summaries (Geometry Matters in Packed 3D Attention,
// project page Ch. 3 "Rotate first, then pool"; paper summary §3.2, §B.5).
//
// One workgroup per (group of 8 consecutive summaries, batch); the summary
// count is padded to Mp = 32*ceil(M/32) and padding slots are written as 0. For each of
// its blocks the workgroup stages the members' memory positions (slot map
// lookups in canonical within-block-slot order) in LDS, then every thread
// accumulates its channel pair of the members' contiguous [H, D] rows in
// fp32, in that order -- so the summaries are the same bits under any
// packing of the tokens. HBM-bound: every K and V element is read once.
//
// Outputs, both blocked so that the matrix-core kernel streams them with
// contiguous 16-byte-per-lane loads:
//   k_sum [B, H, Mp/32, Dp/8, 32, 8]: element (m, d) at [b, h, m/32, d/8, m%32, d%8]
//                                   (Dp = 8*ceil(D/8); padding channels are 0)
//   v_sum [B, H, Mp/8, D, 8]:        element (m, d) at [b, h, m/8, d, m%8]
// Holding 8 consecutive summaries per workgroup makes every v_sum write a
// full 16-byte chunk.
#include "launch.hpp"

namespace pk {

constexpr int kMaxVol = 512;  // members staged in LDS per pass

template <typename T>
__global__ __launch_bounds__(256) void k_summarize(Geo g, const void *geom, const T *k,
                                                   const T *v, T *ks, T *vsb) {
  __shared__ int s_slot[kMaxVol];
  const int g8 = blockIdx.x, b = blockIdx.y;
  const int Mp = (g.M + 31) / 32 * 32;
  const int Dp = (g.D + 7) / 8 * 8;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int half = g.D / 2, da = g.D / 3, npair = g.H * half;
  // Each thread keeps up to 2 channel pairs (npair <= 2 * blockDim.x) for
  // the 8 blocks of its group.
  float ka[2][8][2], va[2][8][2];
  int cnt[8];
#pragma unroll
  for (int u = 0; u < 2; u++)
#pragma unroll
    for (int s = 0; s < 8; s++) ka[u][s][0] = ka[u][s][1] = va[u][s][0] = va[u][s][1] = 0.f;

  auto origin = [&](int m, int *o) {
    o[0] = (m / (g.My * g.Mx)) * g.bz;
    o[1] = ((m / g.Mx) % g.My) * g.by;
    o[2] = (m % g.Mx) * g.bx;
  };
  auto member_slot = [&](int m, int rr) {
    int o[3];
    origin(m, o);
    const int z = o[0] + rr / (g.by * g.bx), y = o[1] + (rr / g.bx) % g.by, x = o[2] + rr % g.bx;
    return (z < g.Z && y < g.Y && x < g.X) ? slot[site_of(g, z, y, x)] : -1;
  };
  // adds member rr (memory position j) of block m into accumulator s
  auto accumulate = [&](int s, int m, int rr, int j) {
    int o[3];
    origin(m, o);
    const int c3[3] = {o[0] + rr / (g.by * g.bx), o[1] + (rr / g.bx) % g.by, o[2] + rr % g.bx};
    const int64_t row = ((int64_t)b * g.N + j) * g.H * g.D;
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int t = threadIdx.x + u * blockDim.x;
      if (t < npair) {
        const int h = t / half, d0 = 2 * (t % half);
        const int a = d0 / da, p = (d0 % da) / 2;
        const T *kp = k + row + h * g.D + d0;
        const T *vp = v + row + h * g.D + d0;
        float k0 = to_f32(kp[0]), k1 = to_f32(kp[1]);
        rotate(k0, k1, rope_cs(tab, g, a, c3[a], p));
#pragma unroll
        for (int ss = 0; ss < 8; ss++)
          if (ss == s) {
            ka[u][ss][0] += k0;
            ka[u][ss][1] += k1;
            va[u][ss][0] += to_f32(vp[0]);
            va[u][ss][1] += to_f32(vp[1]);
          }
      }
    }
  };

#pragma unroll
  for (int s = 0; s < 8; s++) cnt[s] = 0;
  if (8 * g.vol <= kMaxVol) {
    // stage the members of all 8 blocks at once
    for (int idx = threadIdx.x; idx < 8 * g.vol; idx += blockDim.x) {
      const int m = 8 * g8 + idx / g.vol;
      s_slot[idx] = m < g.M ? member_slot(m, idx % g.vol) : -1;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const int m = 8 * g8 + s;
#pragma unroll 4
      for (int r = 0; r < g.vol; r++) {
        const int j = s_slot[s * g.vol + r];
        if (j < 0) continue;
        cnt[s]++;
        accumulate(s, m, r, j);
      }
    }
  } else {
    // large blocks: one block at a time, members in chunks
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const int m = 8 * g8 + s;
      if (m >= g.M) continue;  // uniform
      for (int r0 = 0; r0 < g.vol; r0 += kMaxVol) {
        const int nr = min(kMaxVol, g.vol - r0);
        __syncthreads();
        for (int r = threadIdx.x; r < nr; r += blockDim.x) s_slot[r] = member_slot(m, r0 + r);
        __syncthreads();
        for (int r = 0; r < nr; r++) {
          const int j = s_slot[r];
          if (j < 0) continue;
          cnt[s]++;
          accumulate(s, m, r0 + r, j);
        }
      }
    }
  }

#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int t = threadIdx.x + u * blockDim.x;
    if (t >= npair) continue;
    const int h = t / half, d0 = 2 * (t % half);
    // mean = sum / count (a division, as in the definition); empty -> 0
    float km[8][2], vm[8][2];
#pragma unroll
    for (int s = 0; s < 8; s++)
#pragma unroll
      for (int c = 0; c < 2; c++) {
        km[s][c] = cnt[s] > 0 ? ka[u][s][c] / (float)cnt[s] : 0.0f;
        vm[s][c] = cnt[s] > 0 ? va[u][s][c] / (float)cnt[s] : 0.0f;
      }
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const int m = 8 * g8 + s;
      const int64_t o =
          (((((int64_t)b * g.H + h) * (Mp / 32) + m / 32) * (Dp / 8) + d0 / 8) * 32 + m % 32) * 8 +
          d0 % 8;
      ks[o] = from_f32<T>(km[s][0]);
      ks[o + 1] = from_f32<T>(km[s][1]);
    }
    const int64_t vo = ((((int64_t)b * g.H + h) * (Mp / 8) + g8) * g.D + d0) * 8;
#pragma unroll
    for (int c = 0; c < 2; c++)
#pragma unroll
      for (int s = 0; s < 8; s++) vsb[vo + 8 * c + s] = from_f32<T>(vm[s][c]);
  }
  // padding channels D..Dp of k_sum are zero
  for (int t = threadIdx.x; t < g.H * (Dp - g.D); t += blockDim.x) {
    const int h = t / (Dp - g.D), d = g.D + t % (Dp - g.D);
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const int m = 8 * g8 + s;
      ks[(((((int64_t)b * g.H + h) * (Mp / 32) + m / 32) * (Dp / 8) + d / 8) * 32 + m % 32) * 8 +
         d % 8] = from_f32<T>(0.0f);
    }
  }
}

hipError_t launch_summarize(const Geo &g, int dtype, const void *geom, const void *k,
                            const void *v, void *ks, void *vs, hipStream_t s) {
  const int npair = g.H * g.D / 2;
  const int threads = npair <= 256 ? ((npair + 63) / 64) * 64 : 256;
  if (npair > 2 * threads) return hipErrorInvalidValue;  // host checks H*D <= 1024
  dim3 grid((unsigned)((g.M + 31) / 32 * 4), (unsigned)g.B);
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
