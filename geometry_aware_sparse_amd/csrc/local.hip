// Exact 3x3x3 local attention at grid coordinates (Geometry Matters in Packed
// 3D Attention, project page Ch. 3, Contract 1; paper summary §3.2, §3.5),
// optionally fused with the tokenwise mix (paper summary §3.3).
//
// Queries are tiled in grid space: a workgroup owns a TZ x TY x TX box of
// sites for one (batch, head) and stages the box plus a one-site halo of
// RoPE-rotated keys and raw values in LDS, gathering each site's token
// through the coordinate-to-slot map (so any packing is legal input). One
// thread per query then takes the 27 offsets in canonical order: logits,
// maximum, exp2, weighted sum, all in fp32 -- no neighbour tensor is ever
// written to memory (paper summary §3.5). Off-grid or empty sites are staged
// as zero rows with slot -1 and get weight exactly 0.
//
// Workgroups are dealt to XCDs so that the heads of one box and neighbouring
// boxes share an XCD's L2, which holds the halo re-reads.
#include "launch.hpp"

namespace pk {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int N>
__device__ __forceinline__ void load_n(const T *p, float *out) {
#pragma unroll
  for (int u = 0; u < N; u++) out[u] = to_f32(p[u]);
}

}  // namespace

template <typename T, int D, int TZ, int TY, int TX>
__global__ __launch_bounds__(TZ *TY *TX) void k_local(Geo g, const void *geom, const T *__restrict__ q,
                                                      const T *__restrict__ k,
                                                      const T *__restrict__ v, const T *gate,
                                                      const T *oglob, T *out, int ntz, int nty,
                                                      int ntx) {
  constexpr int HZ = TZ + 2, HY = TY + 2, HX = TX + 2, NH = HZ * HY * HX, NT = TZ * TY * TX;
  constexpr int DA = D / 3;
  // chunk of channels moved per staging step: 8 when it stays inside one axis
  constexpr int CW = (DA % 8 == 0) ? 8 : 2;
  constexpr int PITCH = D + 16 / (int)sizeof(T);  // row pitch in elements (16 B pad)
  __shared__ T sK[NH * PITCH];
  __shared__ T sV[NH * PITCH];
  __shared__ int sSlot[NH];

  const int ntiles = ntz * nty * ntx;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int h = w % g.H;
  const int tile = (w / g.H) % ntiles;
  const int b = w / (g.H * ntiles);
  const int z0 = (tile / (nty * ntx)) * TZ, y0 = ((tile / ntx) % nty) * TY, x0 = (tile % ntx) * TX;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int64_t bN = (int64_t)b * g.N;

  // Stage K~ (rotated) and V of the halo box.
  for (int e = threadIdx.x; e < NH * (D / CW); e += NT) {
    const int hs = e / (D / CW), ch = e % (D / CW);
    const int hz = hs / (HY * HX), hy = (hs / HX) % HY, hx = hs % HX;
    const int z = z0 - 1 + hz, y = y0 - 1 + hy, x = x0 - 1 + hx;
    int j = -1;
    if (z >= 0 && y >= 0 && x >= 0 && z < g.Z && y < g.Y && x < g.X) j = slot[site_of(g, z, y, x)];
    if (ch == 0) sSlot[hs] = j;
    float kv[CW], vv[CW];
    if (j >= 0) {
      const int64_t off = ((bN + j) * g.H + h) * D + ch * CW;
      load_n<T, CW>(k + off, kv);
      load_n<T, CW>(v + off, vv);
      const int c3[3] = {z, y, x};
#pragma unroll
      for (int u = 0; u < CW; u += 2) {
        const int d0 = ch * CW + u, a = d0 / DA, p = (d0 % DA) / 2;
        rotate(kv[u], kv[u + 1], rope_cs(tab, g, a, c3[a], p));
      }
    } else {
#pragma unroll
      for (int u = 0; u < CW; u++) kv[u] = vv[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < CW; u++) {
      sK[hs * PITCH + ch * CW + u] = from_f32<T>(kv[u]);
      sV[hs * PITCH + ch * CW + u] = from_f32<T>(vv[u]);
    }
  }
  __syncthreads();

  const int t = threadIdx.x;
  const int tz = t / (TY * TX), ty = (t / TX) % TY, tx = t % TX;
  const int qs = ((tz + 1) * HY + (ty + 1)) * HX + (tx + 1);
  const int i = sSlot[qs];  // -1 when the query site is off the grid or empty
  if (i < 0) return;
  const int c3[3] = {z0 + tz, y0 + ty, x0 + tx};
  const float qscale = g.scale * kLog2e;

  float qv[D];
  {
    const int64_t off = ((bN + i) * g.H + h) * D;
    load_n<T, D>(q + off, qv);
#pragma unroll
    for (int d0 = 0; d0 < D; d0 += 2) {
      rotate(qv[d0], qv[d0 + 1], rope_cs(tab, g, d0 / DA, c3[d0 / DA], (d0 % DA) / 2));
      qv[d0] *= qscale;
      qv[d0 + 1] *= qscale;
    }
  }

  // logits in log2 units, canonical offset order k = (dz+1)*9 + (dy+1)*3 + dx+1
  float lg[27];
  float mx = -INFINITY;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    const int hs = qs + ((kk / 9) - 1) * HY * HX + (((kk / 3) % 3) - 1) * HX + (kk % 3) - 1;
    const T *kr = sK + hs * PITCH;
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < D; d++) acc += qv[d] * to_f32(kr[d]);
    lg[kk] = sSlot[hs] >= 0 ? acc : -INFINITY;
    mx = fmaxf(mx, lg[kk]);
  }
  float o[D];
#pragma unroll
  for (int d = 0; d < D; d++) o[d] = 0.f;
  float den = 0.f;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    const int hs = qs + ((kk / 9) - 1) * HY * HX + (((kk / 3) % 3) - 1) * HX + (kk % 3) - 1;
    const float p = exp2f(lg[kk] - mx);  // exactly 0 for an invalid neighbour
    den += p;
    const T *vr = sV + hs * PITCH;
#pragma unroll
    for (int d = 0; d < D; d++) o[d] += p * to_f32(vr[d]);
  }
  const float inv = 1.0f / den;
  const int64_t off = ((bN + i) * g.H + h) * D;
  if (gate) {
    const float gl = to_f32(gate[(bN + i) * g.H + h]);
    const float gg = 1.0f / (1.0f + expf(-gl));
    float og[D];
    load_n<T, D>(oglob + off, og);
#pragma unroll
    for (int d = 0; d < D; d++) out[off + d] = from_f32<T>((1.0f - gg) * (o[d] * inv) + gg * og[d]);
  } else {
#pragma unroll
    for (int d = 0; d < D; d++) out[off + d] = from_f32<T>(o[d] * inv);
  }
}

namespace {

template <typename T, int D, int TZ, int TY, int TX>
hipError_t run_local(const Geo &g, const void *geom, const void *q, const void *k, const void *v,
                     const void *gate, const void *og, void *out, hipStream_t s) {
  const int ntz = (g.Z + TZ - 1) / TZ, nty = (g.Y + TY - 1) / TY, ntx = (g.X + TX - 1) / TX;
  const int64_t nwg = (int64_t)g.B * ntz * nty * ntx * g.H;
  hipLaunchKernelGGL((k_local<T, D, TZ, TY, TX>), dim3((unsigned)nwg), dim3(TZ * TY * TX), 0, s,
                     g, geom, static_cast<const T *>(q), static_cast<const T *>(k),
                     static_cast<const T *>(v), static_cast<const T *>(gate),
                     static_cast<const T *>(og), static_cast<T *>(out), ntz, nty, ntx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_local(const Geo &g, int dtype, const void *geom, const void *q, const void *k,
                        const void *v, const void *gate, const void *oglob, void *out,
                        hipStream_t s, bool *supported) {
  *supported = true;
  if (dtype == PACK3D_BF16) {
    switch (g.D) {
      case 6: return run_local<bf16, 6, 4, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
      case 12: return run_local<bf16, 12, 4, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
      case 24: return run_local<bf16, 24, 4, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
      case 48: return run_local<bf16, 48, 4, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
      case 96: return run_local<bf16, 96, 2, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
    }
  } else {
    switch (g.D) {
      case 6: return run_local<float, 6, 4, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
      case 12: return run_local<float, 12, 4, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
      case 24: return run_local<float, 24, 4, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
      case 48: return run_local<float, 48, 2, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
      case 96: return run_local<float, 96, 1, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
    }
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace pk
