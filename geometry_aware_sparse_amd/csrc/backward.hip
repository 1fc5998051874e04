// Backward of the PACK3D forward (Geometry Matters in Packed 3D Attention:
// the operator is trained end to end and its backward follows the forward's
// streamed access pattern, paper summary §1, §3.4). The gradients are the
// chain rule through the forward's steps in reverse:
//
//   mix      g = sigmoid(G): dG = g (1 - g) <dO, O_glob - O_loc>,
//            dO_loc = (1 - g) dO, dO_glob = g dO
//   softmax attention (local over the 3x3x3 neighbours, global over the
//            allowed summaries): dP_j = <dO, v_j>, Delta = sum_j P_j dP_j,
//            dS_j = P_j (dP_j - Delta); dq~ += s sum_j dS_j k_j,
//            dk_j += s dS_j q~, dv_j += P_j dO
//   pooling  each member present receives dk_sum / n_m and dv_sum / n_m
//            (the centre variant routes the key part through R(centre)^T)
//   RoPE     dx = R(c)^T dx~
//
// The kernels here are the generic vector-unit path (every dtype, head dim
// and exclusion reading). launch_backward sends bf16 rows of 48 or 96
// channels to the matrix-core global branch (backward_mfma.hip, without
// exclusion) and the pair-lane local branch (local_bwd.hip) instead. Every
// reduction runs in a fixed order, so results are reproducible and a repack
// of the tokens permutes the gradients bit for bit.
//
//   k_bwd_prep       per (token, query head): rotated query, dO_glob = g dO,
//                    Delta_glob = <dO_glob, O_glob>
//   k_bwd_global_q   per (token, query head): dq~ from the summaries, with
//                    the forward's saved log-sum-exp
//   k_bwd_global_kv  per (summary, KV head): d k_sum and d v_sum, reduced over
//                    every query of the KV head's group in grid-site order
//   k_bwd_local_q    per query site: the local softmax recomputed, dq (both
//                    branches, rotated back), dG, and the local log-sum-exp
//                    and Delta for the key side
//   k_bwd_local_kv   per key site and KV head: the neighbourhood relation is
//                    symmetric, so a key gathers from its <= 27 neighbour
//                    queries (no atomics); then the pooling and RoPE
//                    transposes, and dk, dv are written once
#include "launch.hpp"

namespace pk {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNT = 256;  // threads per workgroup of the per-token kernels
constexpr int kTS = 32;   // summaries (or queries) per LDS tile

// Rotate the pair (x0, x1) by R^T: the rotation by the negative angle.
__device__ __forceinline__ void rotate_t(float &x0, float &x1, float2 cs) {
  float y0 = x0 * cs.x + x1 * cs.y;
  float y1 = -x0 * cs.y + x1 * cs.x;
  x0 = y0;
  x1 = y1;
}

template <typename T, int D>
__device__ __forceinline__ void load_row(const T *p, float *out) {
#pragma unroll
  for (int d = 0; d < D; d++) out[d] = to_f32(p[d]);
}

// (cos, sin) at the centre of block m along axis a, plane p: the table row
// of origin + l, or (for an even extent) row origin + l advanced by the
// half-angle row, as the pooling kernel computes it.
__device__ __forceinline__ float2 centre_cs(const float2 *tab, const Geo &g, int m, int a, int p) {
  const int mz = m / (g.My * g.Mx), my = (m / g.Mx) % g.My, mx = m % g.Mx;
  const int o = a == 0 ? mz * g.bz : (a == 1 ? my * g.by : mx * g.bx);
  const int ext = min(a == 0 ? g.bz : (a == 1 ? g.by : g.bx), (a == 0 ? g.Z : (a == 1 ? g.Y : g.X)) - o);
  float2 t = rope_cs(tab, g, a, o + (ext - 1) / 2, p);
  if ((ext & 1) == 0) {
    const float2 hh = rope_half(tab, g, p);
    t = make_float2(t.x * hh.x - t.y * hh.y, t.y * hh.x + t.x * hh.y);
  }
  return t;
}

__device__ __forceinline__ int members_of(const Geo &g, int m) {
  const int mz = m / (g.My * g.Mx), my = (m / g.Mx) % g.My, mx = m % g.Mx;
  return min(g.bz, g.Z - mz * g.bz) * min(g.by, g.Y - my * g.by) * min(g.bx, g.X - mx * g.bx);
}
}  // namespace

// ---------------------------------------------------------------------------
// Per (token, query head): q~ = R(c) q (fp32, unscaled), dO_glob = g dO and
// Delta_glob = <dO_glob, O_glob>; a token off the grid gets zeros.
template <typename T, int D>
__global__ __launch_bounds__(kNT) void k_bwd_prep(Geo g, const void *geom,
                                                  const int32_t *__restrict__ coords,
                                                  const T *__restrict__ q,
                                                  const T *__restrict__ gate,
                                                  const T *__restrict__ dout,
                                                  const T *__restrict__ oglob, float *qr,
                                                  float *dog, float *delta_g) {
  constexpr int DA = D / 3;
  const int64_t row = (int64_t)blockIdx.x * kNT + threadIdx.x;  // (b, i, h)
  if (row >= (int64_t)g.B * g.N * g.H) return;
  const int i = (int)((row / g.H) % g.N);
  const int c3[3] = {coords[3 * (int64_t)i], coords[3 * (int64_t)i + 1], coords[3 * (int64_t)i + 2]};
  const bool cok = c3[0] >= 0 && c3[1] >= 0 && c3[2] >= 0 && c3[0] < g.Z && c3[1] < g.Y &&
                   c3[2] < g.X;
  const float2 *tab = rope_table(geom, g);
  const float gg = 1.0f / (1.0f + expf(-to_f32(gate[row])));
  float dl = 0.f;
#pragma unroll
  for (int d0 = 0; d0 < D; d0 += 2) {
    float x0 = 0.f, x1 = 0.f;
    if (cok) {
      x0 = to_f32(q[row * D + d0]);
      x1 = to_f32(q[row * D + d0 + 1]);
      rotate(x0, x1, rope_cs(tab, g, d0 / DA, c3[d0 / DA], (d0 % DA) / 2));
    }
    qr[row * D + d0] = x0;
    qr[row * D + d0 + 1] = x1;
    const float e0 = cok ? gg * to_f32(dout[row * D + d0]) : 0.f;
    const float e1 = cok ? gg * to_f32(dout[row * D + d0 + 1]) : 0.f;
    dog[row * D + d0] = e0;
    dog[row * D + d0 + 1] = e1;
    dl += e0 * to_f32(oglob[row * D + d0]) + e1 * to_f32(oglob[row * D + d0 + 1]);
  }
  delta_g[row] = dl;
}

// ---------------------------------------------------------------------------
// Global branch, query side: dq~_i = s sum_m P_im (dP_im - Delta_i) k_sum_m
// with P_im = exp2(t_im - lse_i), t in log2 units (scores scaled by
// s log2 e, as in the forward), dP_im = <dO_glob_i, v_sum_m>. Summaries are
// streamed through LDS in tiles of 32 in block-id order.
template <typename T, int D>
__global__ __launch_bounds__(kNT) void k_bwd_global_q(Geo g, const int32_t *__restrict__ coords,
                                                      const float *__restrict__ qr,
                                                      const float *__restrict__ dog,
                                                      const float *__restrict__ lse,
                                                      const float *__restrict__ delta_g,
                                                      const T *__restrict__ ks,
                                                      const T *__restrict__ vs, float *dqg,
                                                      int ntiles) {
  __shared__ float sK[kTS * D];
  __shared__ float sV[kTS * D];
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = w % ntiles, bh = w / ntiles;
  const int h = bh % g.H, b = bh / g.H;
  const int i = tile * kNT + threadIdx.x;
  const bool active = i < g.N;
  const int Mp = (g.M + 31) / 32 * 32;
  const int64_t bk = (int64_t)b * g.Hkv + h / g.G;
  const int64_t kbase = bk * (Mp / 32), vbase = bk * (Mp / 8);
  const int64_t row = ((int64_t)b * g.N + (active ? i : 0)) * g.H + h;
  const float qscale = g.scale * kLog2e;
  float qv[D], dv[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; d++) qv[d] = dv[d] = 0.f;
  int c3[3] = {0, 0, 0};
  float l = -INFINITY, dl = 0.f;
  if (active) {
    load_row<float, D>(qr + row * D, qv);
    load_row<float, D>(dog + row * D, dv);
    l = lse[row];
    dl = delta_g[row];
    c3[0] = coords[3 * (int64_t)i];
    c3[1] = coords[3 * (int64_t)i + 1];
    c3[2] = coords[3 * (int64_t)i + 2];
  }
  // no attendable summary (or off the grid): the branch output was 0
  const bool live = active && l != -INFINITY;
#pragma unroll
  for (int d = 0; d < D; d++) {
    qv[d] *= qscale;
    acc[d] = 0.f;
  }
  for (int m0 = 0; m0 < g.M; m0 += kTS) {
    const int nm = min(kTS, g.M - m0);
    __syncthreads();
    for (int e = threadIdx.x; e < nm * D; e += kNT) {
      const int m = m0 + e / D, d = e % D;
      sK[e] = to_f32(ks[(((kbase + m / 32) * ((D + 7) / 8) + d / 8) * 32 + m % 32) * 8 + d % 8]);
      sV[e] = to_f32(vs[((vbase + m / 8) * D + d) * 8 + m % 8]);
    }
    __syncthreads();
    if (!live) continue;
    for (int u = 0; u < nm; u++) {
      if (summary_excluded(g, c3[0], c3[1], c3[2], m0 + u)) continue;
      float t = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; d++) {
        t += qv[d] * sK[u * D + d];
        dp += dv[d] * sV[u * D + d];
      }
      const float ds = exp2f(t - l) * (dp - dl);
#pragma unroll
      for (int d = 0; d < D; d++) acc[d] += ds * sK[u * D + d];
    }
  }
  if (!active) return;
#pragma unroll
  for (int d = 0; d < D; d++) dqg[row * D + d] = g.scale * acc[d];
}

// ---------------------------------------------------------------------------
// Global branch, summary side: for summary m of KV head hk,
//   d k_sum_m = s sum_{h in group} sum_i P_im (dP_im - Delta_i) q~_i
//   d v_sum_m = sum_{h in group} sum_i P_im dO_glob_i
// One thread per summary; queries stream through LDS in tiles of 32 in
// (head, grid site) order -- sites in raster order, each mapped to its token
// through the slot map -- so the sums do not depend on the packing.
template <int D>
__global__ __launch_bounds__(64) void k_bwd_global_kv(Geo g, const void *geom,
                                                      const float *__restrict__ qr,
                                                      const float *__restrict__ dog,
                                                      const float *__restrict__ lse,
                                                      const float *__restrict__ delta_g,
                                                      const void *__restrict__ ks_raw,
                                                      const void *__restrict__ vs_raw, int bf,
                                                      float *dks, float *dvs, int mtiles) {
  constexpr int PD = D + 1;  // odd pitch: a thread's own row walks distinct banks
  __shared__ float sKm[64 * PD], sVm[64 * PD];
  __shared__ float sQ[kTS * D], sO[kTS * D], sL[kTS], sDl[kTS];
  __shared__ int sC[kTS * 3], sTok[kTS];
  const int32_t *slot = slot_map(geom, g);
  const int mt = blockIdx.x % mtiles, bk = blockIdx.x / mtiles;  // bk = b * Hkv + hk
  const int b = bk / g.Hkv, hk = bk % g.Hkv;
  const int m = mt * 64 + threadIdx.x;
  const bool mine = m < g.M;
  const int Mp = (g.M + 31) / 32 * 32;
  for (int e = threadIdx.x; e < 64 * D; e += 64) {
    const int u = e / D, d = e % D, mm = min(mt * 64 + u, g.M - 1);
    const int64_t ko = ((((int64_t)bk * (Mp / 32) + mm / 32) * ((D + 7) / 8) + d / 8) * 32 + mm % 32) * 8 + d % 8;
    const int64_t vo = (((int64_t)bk * (Mp / 8) + mm / 8) * D + d) * 8 + mm % 8;
    sKm[u * PD + d] = bf ? (float)static_cast<const bf16 *>(ks_raw)[ko] : static_cast<const float *>(ks_raw)[ko];
    sVm[u * PD + d] = bf ? (float)static_cast<const bf16 *>(vs_raw)[vo] : static_cast<const float *>(vs_raw)[vo];
  }
  const float qscale = g.scale * kLog2e;
  float ak[D], av[D];
#pragma unroll
  for (int d = 0; d < D; d++) ak[d] = av[d] = 0.f;
  for (int h = hk * g.G; h < (hk + 1) * g.G; h++) {
    for (int i0 = 0; i0 < g.N; i0 += kTS) {
      const int ni = min(kTS, g.N - i0);  // sites i0 .. i0 + ni (N = Z*Y*X)
      __syncthreads();
      for (int e = threadIdx.x; e < ni; e += 64) {
        const int site = i0 + e;
        const int i = slot_get(g, slot, site);
        const int64_t row = ((int64_t)b * g.N + max(i, 0)) * g.H + h;
        sTok[e] = i;
        sL[e] = i >= 0 ? lse[row] : -INFINITY;  // an empty site takes no part
        sDl[e] = i >= 0 ? delta_g[row] : 0.f;
        sC[3 * e] = site / (g.Y * g.X);
        sC[3 * e + 1] = (site / g.X) % g.Y;
        sC[3 * e + 2] = site % g.X;
      }
      __syncthreads();
      for (int e = threadIdx.x; e < ni * D; e += 64) {
        const int i = max(sTok[e / D], 0);
        const int64_t row = ((int64_t)b * g.N + i) * g.H + h;
        sQ[e] = qr[row * D + e % D];
        sO[e] = dog[row * D + e % D];
      }
      __syncthreads();
      if (!mine) continue;
      for (int u = 0; u < ni; u++) {
        const float l = sL[u];
        if (l == -INFINITY || summary_excluded(g, sC[3 * u], sC[3 * u + 1], sC[3 * u + 2], m))
          continue;
        float t = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < D; d++) {
          t += (sQ[u * D + d] * qscale) * sKm[threadIdx.x * PD + d];
          dp += sO[u * D + d] * sVm[threadIdx.x * PD + d];
        }
        const float p = exp2f(t - l);
        const float ds = p * (dp - sDl[u]);
#pragma unroll
        for (int d = 0; d < D; d++) {
          ak[d] += ds * sQ[u * D + d];
          av[d] += p * sO[u * D + d];
        }
      }
    }
  }
  if (!mine) return;
  const int64_t o = ((int64_t)bk * g.M + m) * D;
#pragma unroll
  for (int d = 0; d < D; d++) {
    dks[o + d] = g.scale * ak[d];
    dvs[o + d] = av[d];
  }
}

// ---------------------------------------------------------------------------
// Local branch, query side. A workgroup owns a TZ x TY x TX box of query
// sites for one (batch, query head) and stages the box plus its one-site halo
// of rotated keys (rounded to T, as the forward stages them) and values of
// the head's KV head. Per query: logits in log2 units, maximum, exp2, then
//   u_j = <dO, v_j>, <dO, O_loc> = sum_j P_j u_j, dP_j = (1 - g) u_j,
//   Delta = sum_j P_j dP_j, dS_j = P_j (dP_j - Delta),
//   dq = R^T (s sum_j dS_j k~_j + dq~_glob), dG = g (1 - g) (<dO, O_glob> - <dO, O_loc>),
// and the local log-sum-exp (log2 units) and Delta for the key side.
template <typename T, int D, int TZ, int TY, int TX>
__global__ __launch_bounds__(TZ *TY *TX) void k_bwd_local_q(
    Geo g, const void *geom, const T *__restrict__ q, const T *__restrict__ k,
    const T *__restrict__ v, const T *__restrict__ gate, const T *__restrict__ dout,
    const T *__restrict__ oglob, const float *__restrict__ dqg, T *dq, T *dgate, float *lse_l,
    float *delta_l, int ntz, int nty, int ntx) {
  constexpr int HZ = TZ + 2, HY = TY + 2, HX = TX + 2, NH = HZ * HY * HX, NT = TZ * TY * TX;
  constexpr int DA = D / 3;
  constexpr int PITCH = D + 16 / (int)sizeof(T);
  __shared__ T sK[NH * PITCH];
  __shared__ T sV[NH * PITCH];
  __shared__ int sSlot[NH];
  const int ntiles = ntz * nty * ntx;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int h = w % g.H, tile = (w / g.H) % ntiles, b = w / (g.H * ntiles);
  const int hk = h / g.G;
  const int z0 = (tile / (nty * ntx)) * TZ, y0 = ((tile / ntx) % nty) * TY, x0 = (tile % ntx) * TX;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int64_t bN = (int64_t)b * g.N;

  for (int e = threadIdx.x; e < NH * D / 2; e += NT) {
    const int hs = e / (D / 2), d0 = 2 * (e % (D / 2));
    const int hz = hs / (HY * HX), hy = (hs / HX) % HY, hx = hs % HX;
    const int z = z0 - 1 + hz, y = y0 - 1 + hy, x = x0 - 1 + hx;
    int j = -1;
    if (z >= 0 && y >= 0 && x >= 0 && z < g.Z && y < g.Y && x < g.X) j = slot_get(g, slot, site_of(g, z, y, x));
    if (d0 == 0) sSlot[hs] = j;
    float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
    if (j >= 0) {
      const int64_t off = ((bN + j) * g.Hkv + hk) * D + d0;
      k0 = to_f32(k[off]);
      k1 = to_f32(k[off + 1]);
      v0 = to_f32(v[off]);
      v1 = to_f32(v[off + 1]);
      const int c3[3] = {z, y, x};
      rotate(k0, k1, rope_cs(tab, g, d0 / DA, c3[d0 / DA], (d0 % DA) / 2));
    }
    sK[hs * PITCH + d0] = from_f32<T>(k0);
    sK[hs * PITCH + d0 + 1] = from_f32<T>(k1);
    sV[hs * PITCH + d0] = from_f32<T>(v0);
    sV[hs * PITCH + d0 + 1] = from_f32<T>(v1);
  }
  __syncthreads();

  const int t = threadIdx.x;
  const int tz = t / (TY * TX), ty = (t / TX) % TY, tx = t % TX;
  const int qs = ((tz + 1) * HY + (ty + 1)) * HX + (tx + 1);
  const int i = sSlot[qs];
  if (i < 0) return;
  const int c3[3] = {z0 + tz, y0 + ty, x0 + tx};
  const float qscale = g.scale * kLog2e;
  const int64_t row = (bN + i) * g.H + h;

  float qv[D];
  load_row<T, D>(q + row * D, qv);
#pragma unroll
  for (int d0 = 0; d0 < D; d0 += 2)
    rotate(qv[d0], qv[d0 + 1], rope_cs(tab, g, d0 / DA, c3[d0 / DA], (d0 % DA) / 2));
  auto nb = [&](int kk) {
    return qs + ((kk / 9) - 1) * HY * HX + (((kk / 3) % 3) - 1) * HX + (kk % 3) - 1;
  };
  float lg[27];
  float mx = -INFINITY;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    const T *kr = sK + nb(kk) * PITCH;
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < D; d++) acc += qv[d] * to_f32(kr[d]);
    lg[kk] = sSlot[nb(kk)] >= 0 ? acc * qscale : -INFINITY;
    mx = fmaxf(mx, lg[kk]);
  }
  // compiler-only memory barriers between the phases: each phase re-reads
  // its staged rows from LDS instead of keeping 27 rows live in registers
  asm volatile("" ::: "memory");
  float den = 0.f;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    lg[kk] = exp2f(lg[kk] - mx);  // exactly 0 for an invalid neighbour
    den += lg[kk];
  }
  const float inv = 1.0f / den;
  float dov[D];
  load_row<T, D>(dout + row * D, dov);
  const float gg = 1.0f / (1.0f + expf(-to_f32(gate[row])));
  float u[27];
  float dol = 0.f;  // <dO, O_loc>
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    lg[kk] *= inv;
    const T *vr = sV + nb(kk) * PITCH;
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < D; d++) acc += dov[d] * to_f32(vr[d]);
    u[kk] = acc;
    dol += lg[kk] * acc;
  }
  const float delta = (1.0f - gg) * dol;
  asm volatile("" ::: "memory");
  float dqv[D];
#pragma unroll
  for (int d = 0; d < D; d++) dqv[d] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    const float ds = lg[kk] * ((1.0f - gg) * u[kk] - delta);
    const T *kr = sK + nb(kk) * PITCH;
#pragma unroll
    for (int d = 0; d < D; d++) dqv[d] += ds * to_f32(kr[d]);
  }
  float dog_o = 0.f;  // <dO, O_glob>
  {
    float og[D];
    load_row<T, D>(oglob + row * D, og);
#pragma unroll
    for (int d = 0; d < D; d++) dog_o += dov[d] * og[d];
  }
#pragma unroll
  for (int d0 = 0; d0 < D; d0 += 2) {
    float x0 = g.scale * dqv[d0] + dqg[row * D + d0];
    float x1 = g.scale * dqv[d0 + 1] + dqg[row * D + d0 + 1];
    rotate_t(x0, x1, rope_cs(tab, g, d0 / DA, c3[d0 / DA], (d0 % DA) / 2));
    dq[row * D + d0] = from_f32<T>(x0);
    dq[row * D + d0 + 1] = from_f32<T>(x1);
  }
  dgate[row] = from_f32<T>(gg * (1.0f - gg) * (dog_o - dol));
  lse_l[row] = mx + log2f(den);
  delta_l[row] = delta;
}

// ---------------------------------------------------------------------------
// Local branch, key side, plus the pooling and RoPE transposes. A workgroup
// owns a box of key sites for one (batch, KV head); for every query head of
// the group it stages the box plus halo of raw queries and output gradients
// with each site's (1 - g), local log-sum-exp and Delta. A key j visits its
// <= 27 neighbours i (i is a neighbour of j exactly when j is one of i), in
// the fixed offset order, and rebuilds P_ij and dS_ij from the query side's
// statistics:
//   dk~_j += s dS_ij q~_i,   dv_j += P_ij (1 - g_i) dO_i;
// then the block's d k_sum / n_m and d v_sum / n_m, and dk = R(c_j)^T dk~_j.
template <typename T, int D, int TZ, int TY, int TX, bool CENTRE>
__global__ __launch_bounds__(TZ *TY *TX) void k_bwd_local_kv(
    Geo g, const void *geom, const T *__restrict__ q, const T *__restrict__ k,
    const T *__restrict__ v, const T *__restrict__ gate, const T *__restrict__ dout,
    const float *__restrict__ lse_l, const float *__restrict__ delta_l,
    const float *__restrict__ dks, const float *__restrict__ dvs, T *dk, T *dv, int ntz, int nty,
    int ntx) {
  constexpr int HZ = TZ + 2, HY = TY + 2, HX = TX + 2, NH = HZ * HY * HX, NT = TZ * TY * TX;
  constexpr int DA = D / 3;
  constexpr int PITCH = D + 16 / (int)sizeof(T);
  __shared__ T sQ[NH * PITCH];
  __shared__ T sO[NH * PITCH];
  __shared__ float sG[NH], sL[NH], sDl[NH];
  __shared__ int sSlot[NH];
  const int ntiles = ntz * nty * ntx;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int hk = w % g.Hkv, tile = (w / g.Hkv) % ntiles, b = w / (g.Hkv * ntiles);
  const int z0 = (tile / (nty * ntx)) * TZ, y0 = ((tile / ntx) % nty) * TY, x0 = (tile % ntx) * TX;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int64_t bN = (int64_t)b * g.N;
  const float qscale = g.scale * kLog2e;

  const int t = threadIdx.x;
  const int tz = t / (TY * TX), ty = (t / TX) % TY, tx = t % TX;
  const int ks_ = ((tz + 1) * HY + (ty + 1)) * HX + (tx + 1);
  const int c3[3] = {z0 + tz, y0 + ty, x0 + tx};
  const bool on = c3[0] < g.Z && c3[1] < g.Y && c3[2] < g.X;
  const int j = on ? slot_get(g, slot, site_of(g, c3[0], c3[1], c3[2])) : -1;
  const int64_t jrow = (bN + max(j, 0)) * g.Hkv + hk;
  // own key, rotated and rounded to T exactly as the query side staged it
  float kv[D], vv[D];
  load_row<T, D>(k + jrow * D, kv);
  load_row<T, D>(v + jrow * D, vv);
#pragma unroll
  for (int d0 = 0; d0 < D; d0 += 2) {
    rotate(kv[d0], kv[d0 + 1], rope_cs(tab, g, d0 / DA, on ? c3[d0 / DA] : 0, (d0 % DA) / 2));
    kv[d0] = to_f32(from_f32<T>(kv[d0]));
    kv[d0 + 1] = to_f32(from_f32<T>(kv[d0 + 1]));
  }
  float dkv[D], dvv[D];
#pragma unroll
  for (int d = 0; d < D; d++) dkv[d] = dvv[d] = 0.f;

  for (int h = hk * g.G; h < (hk + 1) * g.G; h++) {
    __syncthreads();  // the previous head's stage is no longer read
    for (int e = threadIdx.x; e < NH * D; e += NT) {
      const int hs = e / D, d = e % D;
      const int hz = hs / (HY * HX), hy = (hs / HX) % HY, hx = hs % HX;
      const int z = z0 - 1 + hz, y = y0 - 1 + hy, x = x0 - 1 + hx;
      int i = -1;
      if (z >= 0 && y >= 0 && x >= 0 && z < g.Z && y < g.Y && x < g.X) i = slot_get(g, slot, site_of(g, z, y, x));
      const int64_t row = (bN + max(i, 0)) * g.H + h;
      sQ[hs * PITCH + d] = i >= 0 ? q[row * D + d] : from_f32<T>(0.f);
      sO[hs * PITCH + d] = i >= 0 ? dout[row * D + d] : from_f32<T>(0.f);
      if (d == 0) {
        sSlot[hs] = i;
        sG[hs] = i >= 0 ? 1.0f - 1.0f / (1.0f + expf(-to_f32(gate[row]))) : 0.f;
        sL[hs] = i >= 0 ? lse_l[row] : 0.f;
        sDl[hs] = i >= 0 ? delta_l[row] : 0.f;
      }
    }
    __syncthreads();
    if (j < 0) continue;
#pragma unroll 1
    for (int kk = 0; kk < 27; kk++) {
      const int hs = ks_ + ((kk / 9) - 1) * HY * HX + (((kk / 3) % 3) - 1) * HX + (kk % 3) - 1;
      if (sSlot[hs] < 0) continue;
      const int ci[3] = {c3[0] + kk / 9 - 1, c3[1] + (kk / 3) % 3 - 1, c3[2] + kk % 3 - 1};
      float qv[D];
      load_row<T, D>(sQ + hs * PITCH, qv);
#pragma unroll
      for (int d0 = 0; d0 < D; d0 += 2)
        rotate(qv[d0], qv[d0 + 1], rope_cs(tab, g, d0 / DA, ci[d0 / DA], (d0 % DA) / 2));
      float s = 0.f, u = 0.f;
#pragma unroll
      for (int d = 0; d < D; d++) {
        s += qv[d] * kv[d];
        u += to_f32(sO[hs * PITCH + d]) * vv[d];
      }
      const float p = exp2f(s * qscale - sL[hs]);
      const float og = sG[hs];  // 1 - g_i
      const float ds = p * (og * u - sDl[hs]);
#pragma unroll
      for (int d = 0; d < D; d++) {
        dkv[d] += ds * qv[d];
        dvv[d] += p * og * to_f32(sO[hs * PITCH + d]);
      }
    }
  }
  if (j < 0) return;
  // pooling transpose: this token's block gradient over its member count
  const int m = block_of(g, c3[0], c3[1], c3[2]);
  const float inv_n = 1.0f / (float)members_of(g, m);
  const int64_t so = (((int64_t)b * g.Hkv + hk) * g.M + m) * D;
#pragma unroll
  for (int d = 0; d < D; d++) {
    dkv[d] *= g.scale;
    if (!CENTRE) dkv[d] += dks[so + d] * inv_n;
    dvv[d] += dvs[so + d] * inv_n;
  }
#pragma unroll
  for (int d0 = 0; d0 < D; d0 += 2) {
    const int a = d0 / DA, p = (d0 % DA) / 2;
    float x0 = dkv[d0], x1 = dkv[d0 + 1];
    rotate_t(x0, x1, rope_cs(tab, g, a, c3[a], p));
    if (CENTRE) {
      float y0 = dks[so + d0] * inv_n, y1 = dks[so + d0 + 1] * inv_n;
      rotate_t(y0, y1, centre_cs(tab, g, m, a, p));
      x0 += y0;
      x1 += y1;
    }
    dk[jrow * D + d0] = from_f32<T>(x0);
    dk[jrow * D + d0 + 1] = from_f32<T>(x1);
  }
#pragma unroll
  for (int d = 0; d < D; d++) dv[jrow * D + d] = from_f32<T>(dvv[d]);
}

// ---------------------------------------------------------------------------
namespace {

// Global branch on the vector units: prep, query side, summary side.
template <typename T, int D>
hipError_t run_global_bwd_valu(const Geo &g, const BwdArgs &a, hipStream_t s) {
  const int64_t rows = (int64_t)g.B * g.N * g.H;
  hipLaunchKernelGGL((k_bwd_prep<T, D>), dim3((unsigned)((rows + kNT - 1) / kNT)), dim3(kNT), 0, s,
                     g, a.geom, a.coords, static_cast<const T *>(a.q), static_cast<const T *>(a.gate),
                     static_cast<const T *>(a.dout), static_cast<const T *>(a.oglob), a.qr, a.dog,
                     a.delta_g);
  if (hipError_t e = hipGetLastError()) return e;
  const int ntiles = (g.N + kNT - 1) / kNT;
  hipLaunchKernelGGL((k_bwd_global_q<T, D>), dim3((unsigned)(ntiles * g.B * g.H)), dim3(kNT), 0, s,
                     g, a.coords, a.qr, a.dog, a.lse_g, a.delta_g, static_cast<const T *>(a.ks),
                     static_cast<const T *>(a.vs), a.dqg, ntiles);
  if (hipError_t e = hipGetLastError()) return e;
  const int mtiles = (g.M + 63) / 64;
  hipLaunchKernelGGL((k_bwd_global_kv<D>), dim3((unsigned)(mtiles * g.B * g.Hkv)), dim3(64), 0, s, g,
                     a.geom, a.qr, a.dog, a.lse_g, a.delta_g, a.ks, a.vs, (int)(sizeof(T) == 2),
                     a.dks, a.dvs, mtiles);
  return hipGetLastError();
}

// Local branch on the vector units: query side, then key side.
template <typename T, int D, int TZ, int TY, int TX>
hipError_t run_local_bwd_valu(const Geo &g, const BwdArgs &a, hipStream_t s) {
  const int ntz = (g.Z + TZ - 1) / TZ, nty = (g.Y + TY - 1) / TY, ntx = (g.X + TX - 1) / TX;
  hipLaunchKernelGGL((k_bwd_local_q<T, D, TZ, TY, TX>), dim3((unsigned)(g.B * ntz * nty * ntx * g.H)),
                     dim3(TZ * TY * TX), 0, s, g, a.geom, static_cast<const T *>(a.q),
                     static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                     static_cast<const T *>(a.gate), static_cast<const T *>(a.dout),
                     static_cast<const T *>(a.oglob), a.dqg, static_cast<T *>(a.dq),
                     static_cast<T *>(a.dgate), a.lse_l, a.delta_l, ntz, nty, ntx);
  if (hipError_t e = hipGetLastError()) return e;
  auto kv = (g.flags & PACK3D_SUMMARY_CENTRE) ? k_bwd_local_kv<T, D, TZ, TY, TX, true>
                                               : k_bwd_local_kv<T, D, TZ, TY, TX, false>;
  hipLaunchKernelGGL(kv, dim3((unsigned)(g.B * ntz * nty * ntx * g.Hkv)), dim3(TZ * TY * TX), 0, s, g,
                     a.geom, static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                     static_cast<const T *>(a.v), static_cast<const T *>(a.gate),
                     static_cast<const T *>(a.dout), a.lse_l, a.delta_l, a.dks, a.dvs,
                     static_cast<T *>(a.dk), static_cast<T *>(a.dv), ntz, nty, ntx);
  return hipGetLastError();
}

// The whole backward after the geometry and the summaries: global branch
// (matrix cores when prepared for, else vector units), then local branch
// (pair lanes for bf16 rows of 48 or 96 channels, else vector units).
template <typename T, int D, int TZ, int TY, int TX>
hipError_t run_backward_t(const Geo &g, const BwdArgs &a, hipStream_t s) {
  if (hipError_t e = a.mfma ? launch_bwd_global_mfma(g, a, *a.mfma, s)
                            : run_global_bwd_valu<T, D>(g, a, s))
    return e;
  if (a.events) {  // NULL entries are skipped
    if (a.events[3])
      if (hipError_t e = hipEventRecord(static_cast<hipEvent_t>(a.events[3]), s)) return e;
    if (a.events[4])
      if (hipError_t e = hipEventRecord(static_cast<hipEvent_t>(a.events[4]), s)) return e;
  }
  if (hipError_t e = bwd_local_pair_supported(g, sizeof(T) == 2 ? PACK3D_BF16 : PACK3D_F32)
                         ? launch_bwd_local_pair(g, a, s)
                         : run_local_bwd_valu<T, D, TZ, TY, TX>(g, a, s))
    return e;
  // the kernels above reach tokens through the slot map only: the gradient
  // rows of a token that takes no part are zero
  void *rows[4] = {a.dq, a.dk, a.dv, a.dgate};
  const int len[4] = {g.H * g.D, g.Hkv * g.D, g.Hkv * g.D, g.H};
  return launch_zero_absent(g, (int)sizeof(T), a.geom, a.coords, rows, len, s);
}

}  // namespace

hipError_t launch_backward(const Geo &g, int dtype, const BwdArgs &a, hipStream_t s,
                           bool *supported) {
  *supported = true;
  if (dtype == PACK3D_BF16) {
    switch (g.D) {
      case 6: return run_backward_t<bf16, 6, 4, 4, 8>(g, a, s);
      case 12: return run_backward_t<bf16, 12, 4, 4, 8>(g, a, s);
      case 24: return run_backward_t<bf16, 24, 4, 4, 8>(g, a, s);
      case 48: return run_backward_t<bf16, 48, 4, 4, 4>(g, a, s);
      case 96: return run_backward_t<bf16, 96, 2, 4, 4>(g, a, s);
    }
  } else {
    switch (g.D) {
      case 6: return run_backward_t<float, 6, 4, 4, 8>(g, a, s);
      case 12: return run_backward_t<float, 12, 4, 4, 8>(g, a, s);
      case 24: return run_backward_t<float, 24, 2, 4, 8>(g, a, s);
      case 48: return run_backward_t<float, 48, 2, 4, 4>(g, a, s);
      case 96: return run_backward_t<float, 96, 1, 4, 4>(g, a, s);
    }
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace pk
