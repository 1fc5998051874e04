// Rotate-then-pool block summaries (Geometry Matters in Packed 3D Attention,
// project page Ch. 3 "Rotate first, then pool"; paper summary §3.2, §B.5).
//
// One workgroup per (group of 8 consecutive summaries, batch); the summary
// count is padded to Mp = 32*ceil(M/32) and padding slots are written as 0.
// The workgroup stages the members' memory positions (slot map lookups in
// canonical within-block-slot order) in LDS; a thread owns one block of the
// group and one chunk of CW channels of the token's contiguous [H, D] row,
// and accumulates the members in fp32 in that order -- so the summaries are
// the same bits under any packing of the tokens. HBM-bound: every K and V
// element is read once, with 16-byte loads.
//
// Outputs, both blocked so that the matrix-core kernel streams them with
// contiguous 16-byte-per-lane loads:
//   k_sum [B, H, Mp/32, Dp/8, 32, 8]: element (m, d) at [b, h, m/32, d/8, m%32, d%8]
//                                   (Dp = 8*ceil(D/8); padding channels are 0)
//   v_sum [B, H, Mp/8, D, 8]:        element (m, d) at [b, h, m/8, d, m%8]
// The v_sum means pass through LDS so that each (channel, group) is written
// as one 16-byte chunk.
#include "launch.hpp"

namespace pk {

constexpr int kMaxMembers = 512;  // member slots staged in LDS per pass (8 blocks)

template <typename T, int CW>
__global__ __launch_bounds__(512) void k_summarize(Geo g, const void *geom, const T *k,
                                                   const T *v, T *ks, T *vsb) {
  __shared__ int s_slot[kMaxMembers];
  extern __shared__ float s_vt[];  // [H*D][8] value means for the transposed write
  const int g8 = blockIdx.x, b = blockIdx.y;
  const int Mp = (g.M + 31) / 32 * 32;
  const int Dp = (g.D + 7) / 8 * 8;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int da = g.D / 3;
  const int NC = g.H * g.D / CW;        // channel chunks per token row
  const int CPT = blockDim.x / 8;       // chunk lanes per block
  const int s = threadIdx.x / CPT;      // block of the group owned by this thread
  const int c0 = threadIdx.x % CPT;
  const int m = 8 * g8 + s;
  const int mz = m / (g.My * g.Mx), my = (m / g.Mx) % g.My, mx = m % g.Mx;
  const int o3[3] = {mz * g.bz, my * g.by, mx * g.bx};
  const int64_t bh0 = (int64_t)b * g.H;

  // members of all 8 blocks, in passes of kMaxMembers / 8 per block
  const int per = kMaxMembers / 8;
  // every thread runs the same number of rounds (the barriers below need it)
  const int rounds = (NC + CPT - 1) / CPT;  // usually 1
  for (int rd = 0; rd < rounds; rd++) {
    const int c = c0 + rd * CPT;
    const bool act = c < NC;
    const int h = act ? (c * CW) / g.D : 0, d0 = act ? (c * CW) % g.D : 0;
    float ka[CW], va[CW];
#pragma unroll
    for (int u = 0; u < CW; u++) ka[u] = va[u] = 0.f;
    int cnt = 0;
    for (int r0 = 0; r0 < g.vol; r0 += per) {
      const int nr = min(per, g.vol - r0);
      __syncthreads();
      for (int e = threadIdx.x; e < 8 * nr; e += blockDim.x) {
        const int ss = e / nr, rr = r0 + e % nr, mm = 8 * g8 + ss;
        int j = -1;
        if (mm < g.M) {
          const int z = (mm / (g.My * g.Mx)) * g.bz + rr / (g.by * g.bx);
          const int y = ((mm / g.Mx) % g.My) * g.by + (rr / g.bx) % g.by;
          const int x = (mm % g.Mx) * g.bx + rr % g.bx;
          if (z < g.Z && y < g.Y && x < g.X) j = slot[site_of(g, z, y, x)];
        }
        s_slot[e] = j;
      }
      __syncthreads();
#pragma unroll 4
      for (int r = 0; r < nr; r++) {
        const int j = s_slot[s * nr + r];
        if (j < 0 || !act) continue;
        cnt++;
        const int rr = r0 + r;
        const int c3[3] = {o3[0] + rr / (g.by * g.bx), o3[1] + (rr / g.bx) % g.by, o3[2] + rr % g.bx};
        const int64_t off = (((int64_t)b * g.N + j) * g.H + h) * g.D + d0;
        float kx[CW], vx[CW];
        if constexpr (CW == 8 && sizeof(T) == 2) {
          const bf16x8 kr = *reinterpret_cast<const bf16x8 *>(k + off);
          const bf16x8 vr = *reinterpret_cast<const bf16x8 *>(v + off);
#pragma unroll
          for (int u = 0; u < 8; u++) {
            kx[u] = (float)kr[u];
            vx[u] = (float)vr[u];
          }
        } else {
#pragma unroll
          for (int u = 0; u < CW; u++) {
            kx[u] = to_f32(k[off + u]);
            vx[u] = to_f32(v[off + u]);
          }
        }
#pragma unroll
        for (int u = 0; u < CW; u += 2) {
          const int dd = d0 + u, a = dd / da;
          rotate(kx[u], kx[u + 1], rope_cs(tab, g, a, c3[a], (dd % da) / 2));
        }
#pragma unroll
        for (int u = 0; u < CW; u++) {
          ka[u] += kx[u];
          va[u] += vx[u];
        }
      }
    }
    if (!act) continue;
    // mean = sum / count (a division, as in the definition); empty -> 0
    const int64_t ko = ((((bh0 + h) * (Mp / 32) + m / 32) * (Dp / 8) + d0 / 8) * 32 + m % 32) * 8;
#pragma unroll
    for (int u = 0; u < CW; u++) {
      ks[ko + (d0 + u) % 8] = from_f32<T>(cnt > 0 ? ka[u] / (float)cnt : 0.0f);
      s_vt[(h * g.D + d0 + u) * 8 + s] = cnt > 0 ? va[u] / (float)cnt : 0.0f;
    }
  }
  __syncthreads();
  // v_sum: one 16-byte (bf16) chunk per (head, channel)
  for (int e = threadIdx.x; e < g.H * g.D; e += blockDim.x) {
    const int h = e / g.D, d = e % g.D;
    T *dst = vsb + (((bh0 + h) * (Mp / 8) + g8) * g.D + d) * 8;
#pragma unroll
    for (int u = 0; u < 8; u++) dst[u] = from_f32<T>(s_vt[e * 8 + u]);
  }
  // padding channels D..Dp of k_sum are zero
  for (int e = threadIdx.x; e < 8 * g.H * (Dp - g.D); e += blockDim.x) {
    const int ss = e / (g.H * (Dp - g.D)), rem = e % (g.H * (Dp - g.D));
    const int h = rem / (Dp - g.D), d = g.D + rem % (Dp - g.D), mm = 8 * g8 + ss;
    ks[((((bh0 + h) * (Mp / 32) + mm / 32) * (Dp / 8) + d / 8) * 32 + mm % 32) * 8 + d % 8] =
        from_f32<T>(0.0f);
  }
}

namespace {
template <typename T, int CW>
hipError_t run_summarize(const Geo &g, const void *geom, const void *k, const void *v, void *ks,
                         void *vs, hipStream_t s) {
  const int NC = g.H * g.D / CW;
  const int cpt = NC < 64 ? NC : 64;  // chunk lanes per block
  const size_t lds = (size_t)g.H * g.D * 8 * sizeof(float);
  dim3 grid((unsigned)((g.M + 31) / 32 * 4), (unsigned)g.B);
  hipLaunchKernelGGL((k_summarize<T, CW>), grid, dim3(8 * cpt), lds, s, g, geom,
                     static_cast<const T *>(k), static_cast<const T *>(v), static_cast<T *>(ks),
                     static_cast<T *>(vs));
  return hipGetLastError();
}
}  // namespace

hipError_t launch_summarize(const Geo &g, int dtype, const void *geom, const void *k,
                            const void *v, void *ks, void *vs, hipStream_t s) {
  // host checks H*D <= 1024, so the transposition buffer stays within 32 KiB
  const bool c8 = g.D % 8 == 0;
  if (dtype == PACK3D_BF16)
    return c8 ? run_summarize<bf16, 8>(g, geom, k, v, ks, vs, s)
              : run_summarize<bf16, 2>(g, geom, k, v, ks, vs, s);
  return c8 ? run_summarize<float, 8>(g, geom, k, v, ks, vs, s)
            : run_summarize<float, 2>(g, geom, k, v, ks, vs, s);
}

}  // namespace pk
