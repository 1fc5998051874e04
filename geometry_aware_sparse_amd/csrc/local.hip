// Exact 3x3x3 local attention at grid coordinates (Geometry Matters in Packed
// 3D Attention, project page Ch. 3, Contract 1; paper summary §3.2, §3.5),
// optionally fused with the tokenwise mix (paper summary §3.3).
//
// Queries are tiled in grid space: a workgroup owns a TZ x TY x TX box of
// sites for one (batch, query head) and stages the box plus a one-site halo
// of RoPE-rotated keys and raw values of that head's KV head in LDS, gathering each site's token
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

  const BoxWork wk = box_work(xcd_remap(blockIdx.x, gridDim.x), g.H, ntz, nty, ntx);
  const int h = wk.h, b = wk.b;
  const int z0 = wk.tz * TZ, y0 = wk.ty * TY, x0 = wk.tx * TX;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int64_t bN = (int64_t)b * g.N;

  // Stage K~ (rotated) and V of the halo box.
  for (int e = threadIdx.x; e < NH * (D / CW); e += NT) {
    const int hs = e / (D / CW), ch = e % (D / CW);
    const int hz = hs / (HY * HX), hy = (hs / HX) % HY, hx = hs % HX;
    const int z = z0 - 1 + hz, y = y0 - 1 + hy, x = x0 - 1 + hx;
    int j = -1;
    if (z >= 0 && y >= 0 && x >= 0 && z < g.Z && y < g.Y && x < g.X) j = slot_get(g, slot, site_of(g, z, y, x));
    if (ch == 0) sSlot[hs] = j;
    float kv[CW], vv[CW];
    if (j >= 0) {
      const int64_t off = ((bN + j) * g.Hkv + h / g.G) * D + ch * CW;  // KV head of query head h
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

// bf16 variant for head dims that are multiples of 48: LPQ = D/24 lanes per
// query; lane hh owns channels a*DA + 8hh .. +7 of each axis a (24 in all).
// RoPE enters through relative angles: the logit of key j for query i is
// <R(c_i) q, R(c_j) k> = <R(c_i - c_j) q, k>, the rotations being planar and
// commuting, and every offset c_j - c_i in the neighbourhood is -1, 0 or +1
// along each axis. So each lane rotates its query slice once by the three
// relative angles of its axis and reads the keys unrotated: keys and values
// both reach LDS by direct loads. Dot products use v_dot2_f32_bf16 on packed
// pairs (the rotated, scaled query is rounded to bf16) and the lanes of a
// query meet through DPP lane swaps; the value sum pairs neighbours (k, k+1)
// so that one v_dot2 accumulates two neighbours for one channel, the pairs
// being formed with v_perm_b32.
// At D = 96 a query takes four lanes, so the box is 2 x 4 x 8 sites: four
// waves and 49 KB of LDS, three workgroups per CU at three waves per SIMD with
// no spill. (A 4 x 4 x 8 box needs 8 waves and 74 KB; two of those fit a CU
// only under a 128-VGPR cap, whose spills cost more than the larger halo.)
template <int D, int TZ, int TY, int TX>
__global__ __launch_bounds__((D / 24) * TZ *TY *TX,
                             D == 96 ? (TZ * TY * TX == 128 ? 4 : 3) : 1) void k_local_pair(
    Geo g, const void *geom, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const bf16 *gate, const bf16 *oglob, bf16 *out, int ntz, int nty,
    int ntx) {
  constexpr int HZ = TZ + 2, HY = TY + 2, HX = TX + 2, NH = HZ * HY * HX, NQ = TZ * TY * TX;
  constexpr int LPQ = D / 24;          // lanes per query
  constexpr int NT = LPQ * NQ;
  constexpr int DA = D / 3;            // channels per axis
  constexpr int PITCH = D;             // LDS row pitch (elements), 16-byte aligned rows
  static_assert(D % 48 == 0 && (LPQ == 2 || LPQ == 4), "head dim 48 or 96");
  static_assert(DA == 8 * LPQ, "each lane owns 8 channels (4 planes) of every axis");
  constexpr int CPS = D / 8;                // 16-byte chunks per staged row
  constexpr int NCK = NH * CPS;             // chunks per staged tensor
  constexpr int RS = (NCK + NT - 1) / NT;   // staging rounds per thread
  // rows are PITCH = D apart, so chunk e of the halo is at element 8e; the
  // arrays are padded to whole rounds so that every lane of every round has
  // a place to write
  // one LDS buffer holds the keys for the logits, then the values for the
  // sums, so that the workgroup needs half the LDS and more of them fit a CU
  __shared__ __attribute__((aligned(16))) bf16 sK[RS * NT * 8];
  const bf16 *sV = sK;
  __shared__ int sSlot[NH];

  const BoxWork wk = box_work(xcd_remap(blockIdx.x, gridDim.x), g.H, ntz, nty, ntx);
  const int h = wk.h, b = wk.b;
  const int z0 = wk.tz * TZ, y0 = wk.ty * TY, x0 = wk.tx * TX;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int64_t bN = (int64_t)b * g.N;
  // slots of the halo sites (-1 off the grid): all loads first, then the LDS
  // writes, one barrier
  {
    constexpr int RSL = (NH + NT - 1) / NT;
    int sv[RSL];
#pragma unroll
    for (int r = 0; r < RSL; r++) {
      const int hs = min((int)threadIdx.x + r * NT, NH - 1);
      const int hz = hs / (HY * HX), hy = (hs / HX) % HY, hx = hs % HX;
      const int z = z0 - 1 + hz, y = y0 - 1 + hy, x = x0 - 1 + hx;
      const bool on = z >= 0 && y >= 0 && x >= 0 && z < g.Z && y < g.Y && x < g.X;
      const int j = slot_get(g, slot, on ? site_of(g, z, y, x) : 0);
      sv[r] = on ? j : -1;
    }
#pragma unroll
    for (int r = 0; r < RSL; r++)
      if ((int)threadIdx.x + r * NT < NH) sSlot[threadIdx.x + r * NT] = sv[r];
  }
  __syncthreads();

  // Every global load of the workgroup goes out before any is waited for:
  // the K chunks straight into LDS (16 bytes per lane), the V chunks into
  // registers (they go into the same LDS buffer once the logits are done),
  // this lane's query slices, the (cos, sin) of one step along each of its
  // planes, and for the fused mix its slices of O_glob and the gate. A site off the grid
  // reads token 0 instead: its logit is replaced by -inf and its weight is
  // exactly 0, so only finiteness matters.
  const int qn = threadIdx.x / LPQ, hh = threadIdx.x % LPQ;
  const int tz = qn / (TY * TX), ty = (qn / TX) % TY, tx = qn % TX;
  const int qs = ((tz + 1) * HY + (ty + 1)) * HX + (tx + 1);
  const int i = sSlot[qs];  // all lanes of a query see the same value
  const int wbase = __builtin_amdgcn_readfirstlane(threadIdx.x & ~63);
  bf16x8 vraw[RS];  // value chunks, held until the keys have been used
#pragma unroll
  for (int r = 0; r < RS; r++) {
    const int e = min((int)threadIdx.x + r * NT, NCK - 1);
    const int hs = e / CPS, ch = e % CPS;
    const int64_t off = ((bN + max(sSlot[hs], 0)) * g.Hkv + h / g.G) * D + ch * 8;  // KV head of h
    __builtin_amdgcn_global_load_lds(k + off, (lds_ptr)&sK[(wbase + r * NT) * 8], 16, 0, 0);
    vraw[r] = *reinterpret_cast<const bf16x8 *>(v + off);
  }
  const int64_t row = ((bN + max(i, 0)) * g.H + h) * D;
  bf16x8 qraw[3], ograw[3];
  float gl = 0.f;
#pragma unroll
  for (int a = 0; a < 3; a++) qraw[a] = *reinterpret_cast<const bf16x8 *>(q + row + a * DA + 8 * hh);
  if (gate) {
#pragma unroll
    for (int a = 0; a < 3; a++)
      ograw[a] = *reinterpret_cast<const bf16x8 *>(oglob + row + a * DA + 8 * hh);
    gl = (float)gate[(bN + max(i, 0)) * g.H + h];
  }
  // one unit step of plane 4hh+u of axis a: the table's row for coordinate 1
  // (an axis one site long has no neighbour along it; its row 0 keeps the
  // unused values finite)
  float2 cs1[3][4];
#pragma unroll
  for (int a = 0; a < 3; a++) {
    const int dim = a == 0 ? g.Z : (a == 1 ? g.Y : g.X);
#pragma unroll
    for (int u = 0; u < 4; u++) cs1[a][u] = rope_cs(tab, g, a, min(1, dim - 1), 4 * hh + u);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's loads have landed
  __syncthreads();
  // every lane runs to the end (the barriers below need the whole
  // workgroup); a query site off the grid stores nothing
  const float qscale = g.scale * kLog2e;

  // qv[a][d + 1]: the query slice of axis a, scaled, rotated by the relative
  // angle of a neighbour at offset d along a, R(-d theta), rounded to bf16
  bf16x2 qv[3][3][4];
#pragma unroll
  for (int a = 0; a < 3; a++)
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const float x0v = (float)qraw[a][2 * u] * qscale, x1v = (float)qraw[a][2 * u + 1] * qscale;
#pragma unroll
      for (int d = -1; d <= 1; d++) {
        float y0 = x0v, y1 = x1v;
        if (d != 0) rotate(y0, y1, make_float2(cs1[a][u].x, d > 0 ? -cs1[a][u].y : cs1[a][u].y));
        qv[a][d + 1][u][0] = (bf16)y0;
        qv[a][d + 1][u][1] = (bf16)y1;
      }
    }

  // sum over the LPQ lanes of a query (adjacent lanes) with DPP swaps
  auto lane_sum = [&](float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf,
                                                            0xf, false));  // quad_perm 1,0,3,2
    if constexpr (LPQ == 4)
      x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E,
                                                              0xf, 0xf, false));  // 2,3,0,1
    return x;
  };

  // logits (log2 units) in canonical offset order k = (dz+1)*9 + (dy+1)*3 + dx+1
  float lg[27];
  float mx = -INFINITY;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    const int dd[3] = {kk / 9 - 1, (kk / 3) % 3 - 1, kk % 3 - 1};
    const int hs = qs + dd[0] * HY * HX + dd[1] * HX + dd[2];
    const bf16x2 *kr = reinterpret_cast<const bf16x2 *>(sK + hs * PITCH + 8 * hh);
    float acc = 0.f;
#pragma unroll
    for (int a = 0; a < 3; a++)
#pragma unroll
      for (int u = 0; u < 4; u++)
        acc = __builtin_amdgcn_fdot2_f32_bf16(qv[a][dd[a] + 1][u], kr[a * (DA / 2) + u], acc, false);
    acc = lane_sum(acc);
    lg[kk] = sSlot[hs] >= 0 ? acc : -INFINITY;
    mx = fmaxf(mx, lg[kk]);
  }
  // the keys are no longer read: the buffer takes the values
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RS; r++)
    *reinterpret_cast<bf16x8 *>(&sK[((int)threadIdx.x + r * NT) * 8]) = vraw[r];
  float pr[28];
#pragma unroll
  for (int kk = 0; kk < 27; kk++)
    pr[kk] = __builtin_amdgcn_exp2f(lg[kk] - mx);  // exactly 0 for an invalid neighbour
  pr[27] = 0.f;
  __syncthreads();
  // the weights are rounded to bf16 for the value products; the denominator
  // sums the same rounded weights, so the weights used sum to one
  float den = 0.f;
  bf16x2 ones2;
  ones2[0] = ones2[1] = (bf16)1.0f;
  float o[24];  // channel a*DA + 8hh + c at o[8a + c]
#pragma unroll
  for (int d = 0; d < 24; d++) o[d] = 0.f;
  // neighbours in pairs (2j, 2j+1); the last pair's second member has weight 0
#pragma unroll
  for (int kp = 0; kp < 14; kp++) {
    const int k0 = 2 * kp, k1 = kp < 13 ? 2 * kp + 1 : 2 * kp;
    const int hs0 = qs + ((k0 / 9) - 1) * HY * HX + (((k0 / 3) % 3) - 1) * HX + (k0 % 3) - 1;
    const int hs1 = qs + ((k1 / 9) - 1) * HY * HX + (((k1 / 3) % 3) - 1) * HX + (k1 % 3) - 1;
    bf16x2 pp;
    pp[0] = (bf16)pr[2 * kp];
    pp[1] = (bf16)pr[2 * kp + 1];
    den = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, den, false);
    const uint32_t *A = reinterpret_cast<const uint32_t *>(sV + hs0 * PITCH + 8 * hh);
    const uint32_t *Bv = reinterpret_cast<const uint32_t *>(sV + hs1 * PITCH + 8 * hh);
#pragma unroll
    for (int a = 0; a < 3; a++)
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const uint32_t aw = A[a * (DA / 2) + u], bw = Bv[a * (DA / 2) + u];
        // (a.lo, b.lo) and (a.hi, b.hi)
        const uint32_t lo = __builtin_amdgcn_perm(bw, aw, 0x05040100u);
        const uint32_t hi2 = __builtin_amdgcn_perm(bw, aw, 0x07060302u);
        o[8 * a + 2 * u] =
            __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2, lo), o[8 * a + 2 * u], false);
        o[8 * a + 2 * u + 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2, hi2),
                                                               o[8 * a + 2 * u + 1], false);
      }
  }
  const float inv = 1.0f / den;
  if (i < 0) return;
  if (gate) {
    const float gg = 1.0f / (1.0f + expf(-gl));
#pragma unroll
    for (int a = 0; a < 3; a++) {
      const bf16x8 og = ograw[a];
      bf16x8 r;
#pragma unroll
      for (int u = 0; u < 8; u++)
        r[u] = (bf16)((1.0f - gg) * (o[8 * a + u] * inv) + gg * (float)og[u]);
      *reinterpret_cast<bf16x8 *>(out + row + a * DA + 8 * hh) = r;
    }
  } else {
#pragma unroll
    for (int a = 0; a < 3; a++) {
      bf16x8 r;
#pragma unroll
      for (int u = 0; u < 8; u++) r[u] = (bf16)(o[8 * a + u] * inv);
      *reinterpret_cast<bf16x8 *>(out + row + a * DA + 8 * hh) = r;
    }
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

template <int D, int TZ, int TY, int TX>
hipError_t run_local_pair(const Geo &g, const void *geom, const void *q, const void *k,
                          const void *v, const void *gate, const void *og, void *out,
                          hipStream_t s) {
  const int ntz = (g.Z + TZ - 1) / TZ, nty = (g.Y + TY - 1) / TY, ntx = (g.X + TX - 1) / TX;
  const int64_t nwg = (int64_t)g.B * ntz * nty * ntx * g.H;
  hipLaunchKernelGGL((k_local_pair<D, TZ, TY, TX>), dim3((unsigned)nwg), dim3((D / 24) * TZ * TY * TX), 0,
                     s, g, geom, static_cast<const bf16 *>(q), static_cast<const bf16 *>(k),
                     static_cast<const bf16 *>(v), static_cast<const bf16 *>(gate),
                     static_cast<const bf16 *>(og), static_cast<bf16 *>(out), ntz, nty, ntx);
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
      case 48: return launch_local_tr48(g, geom, q, k, v, gate, oglob, out, s);
      case 96: return run_local_pair<96, 2, 4, 8>(g, geom, q, k, v, gate, oglob, out, s);
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
