// Query-to-summary attention on the fp32 vector units (Geometry Matters in
// Packed 3D Attention, project page Ch. 3, Contract 2; paper summary §3.5).
//
// This is the exact-fp32 path (fp32 tensors) and the path for shapes or
// exclusion readings the matrix-core kernel does not cover. A workgroup owns
// 256 consecutive tokens (packed order) of one (batch, head); each thread
// keeps its rotated, scaled query and its output row in registers and
// streams the summaries through LDS in tiles of 32 with an online softmax in
// block-id order, so no token x summary score matrix exists (paper summary
// §3.5). Every summary read is an LDS broadcast.
#include "launch.hpp"

namespace pk {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTS = 32;   // summaries per LDS tile
constexpr int kNT = 256;  // tokens per workgroup
}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(kNT) void k_global_valu(Geo g, const void *geom,
                                                     const int32_t *__restrict__ coords,
                                                     const T *__restrict__ q,
                                                     const T *__restrict__ ks,
                                                     const T *__restrict__ vs, T *out,
                                                     float *lse, int ntiles) {
  constexpr int DA = D / 3;
  __shared__ float sK[kTS * D];
  __shared__ float sV[kTS * D];
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = w % ntiles;
  const int bh = w / ntiles;
  const int h = bh % g.H, b = bh / g.H;
  const int i = tile * kNT + threadIdx.x;
  const bool active = i < g.N;
  bool cok = false;  // a token that takes no part: zero query, zero output row
  const float2 *tab = rope_table(geom, g);
  const int Mp = (g.M + 31) / 32 * 32;
  const int64_t bk = (int64_t)b * g.Hkv + h / g.G;           // the KV head query head h reads
  const int64_t kbase = bk * (Mp / 32);  // k_sum [B,Hkv,Mp/32,D/8,32,8]
  const int64_t vbase = bk * (Mp / 8);   // v_sum [B,Hkv,Mp/8,D,8]

  float qv[D];
  int c3[3] = {0, 0, 0};
  if (active) {
    c3[0] = coords[3 * (int64_t)i];
    c3[1] = coords[3 * (int64_t)i + 1];
    c3[2] = coords[3 * (int64_t)i + 2];
    cok = takes_part(g, slot_map(geom, g), i, c3[0], c3[1], c3[2]);
  }
  if (cok) {
    const int64_t off = (((int64_t)b * g.N + i) * g.H + h) * D;
    const float qscale = g.scale * kLog2e;
#pragma unroll
    for (int d0 = 0; d0 < D; d0 += 2) {
      float x0 = to_f32(q[off + d0]), x1 = to_f32(q[off + d0 + 1]);
      const int a = d0 / DA;
      rotate(x0, x1, rope_cs(tab, g, a, c3[a], (d0 % DA) / 2));
      qv[d0] = x0 * qscale;
      qv[d0 + 1] = x1 * qscale;
    }
  } else {
#pragma unroll
    for (int d = 0; d < D; d++) qv[d] = 0.f;
  }
  float o[D];
#pragma unroll
  for (int d = 0; d < D; d++) o[d] = 0.f;
  float mx = -INFINITY, den = 0.f;

  for (int m0 = 0; m0 < g.M; m0 += kTS) {
    const int nm = min(kTS, g.M - m0);
    __syncthreads();
    for (int e = threadIdx.x; e < nm * D; e += kNT) {
      const int m = m0 + e / D, d = e % D;
      sK[e] = to_f32(ks[(((kbase + m / 32) * ((D + 7) / 8) + d / 8) * 32 + m % 32) * 8 + d % 8]);
      sV[e] = to_f32(vs[((vbase + m / 8) * D + d) * 8 + m % 8]);
    }
    __syncthreads();
    float lg[kTS];
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kTS; u++) {
      float acc = -INFINITY;
      if (u < nm && cok && !summary_excluded(g, c3[0], c3[1], c3[2], m0 + u)) {
        acc = 0.f;
#pragma unroll
        for (int d = 0; d < D; d++) acc += qv[d] * sK[u * D + d];
      }
      lg[u] = acc;
      tmax = fmaxf(tmax, acc);
    }
    if (tmax == -INFINITY) continue;  // nothing attendable in this tile
    const float mnew = fmaxf(mx, tmax);
    const float alpha = exp2f(mx - mnew);  // 0 while mx is still -inf
    den *= alpha;
#pragma unroll
    for (int d = 0; d < D; d++) o[d] *= alpha;
    mx = mnew;
#pragma unroll
    for (int u = 0; u < kTS; u++) {
      if (u < nm) {  // rows past M hold stale LDS contents
        const float p = exp2f(lg[u] - mx);
        den += p;
#pragma unroll
        for (int d = 0; d < D; d++) o[d] += p * sV[u * D + d];
      }
    }
  }
  if (!active) return;
  const int64_t off = (((int64_t)b * g.N + i) * g.H + h) * D;
  const float inv = (den > 0.f && cok) ? 1.0f / den : 0.f;
#pragma unroll
  for (int d = 0; d < D; d++) out[off + d] = from_f32<T>(o[d] * inv);
  if (lse) lse[((int64_t)b * g.N + i) * g.H + h] = (den > 0.f && cok) ? mx + log2f(den) : -INFINITY;
}

namespace {
template <typename T, int D>
hipError_t run_global_valu(const Geo &g, const void *geom, const int32_t *coords, const void *q,
                           const void *ks, const void *vs, void *out, float *lse, hipStream_t s) {
  const int ntiles = (g.N + kNT - 1) / kNT;
  const int64_t nwg = (int64_t)ntiles * g.B * g.H;
  hipLaunchKernelGGL((k_global_valu<T, D>), dim3((unsigned)nwg), dim3(kNT), 0, s, g, geom, coords,
                     static_cast<const T *>(q), static_cast<const T *>(ks),
                     static_cast<const T *>(vs), static_cast<T *>(out), lse, ntiles);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_global_valu(const Geo &g, int dtype, const void *geom, const int32_t *coords,
                              const void *q, const void *ks, const void *vs, void *out,
                              float *lse, hipStream_t s, bool *supported) {
  *supported = true;
  if (dtype == PACK3D_BF16) {
    switch (g.D) {
      case 6: return run_global_valu<bf16, 6>(g, geom, coords, q, ks, vs, out, lse, s);
      case 12: return run_global_valu<bf16, 12>(g, geom, coords, q, ks, vs, out, lse, s);
      case 24: return run_global_valu<bf16, 24>(g, geom, coords, q, ks, vs, out, lse, s);
      case 48: return run_global_valu<bf16, 48>(g, geom, coords, q, ks, vs, out, lse, s);
      case 96: return run_global_valu<bf16, 96>(g, geom, coords, q, ks, vs, out, lse, s);
    }
  } else {
    switch (g.D) {
      case 6: return run_global_valu<float, 6>(g, geom, coords, q, ks, vs, out, lse, s);
      case 12: return run_global_valu<float, 12>(g, geom, coords, q, ks, vs, out, lse, s);
      case 24: return run_global_valu<float, 24>(g, geom, coords, q, ks, vs, out, lse, s);
      case 48: return run_global_valu<float, 48>(g, geom, coords, q, ks, vs, out, lse, s);
      case 96: return run_global_valu<float, 96>(g, geom, coords, q, ks, vs, out, lse, s);
    }
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace pk
