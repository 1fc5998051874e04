// Exact 3x3x3 local attention, bf16 with head dim 48, with its weighted value
// sums on the matrix cores (Geometry Matters in Packed 3D Attention, project
// page Ch. 3, Contract 1; paper summary §3.2, §3.5), optionally fused with
// the tokenwise mix (paper summary §3.3).
//
// A workgroup owns a 4 x 4 x 8 box of query sites of one (batch, query head)
// and stages the box plus its one-site halo (6 x 6 x 10 sites) of that head's
// KV head through the coordinate-to-slot map, so any packing is legal input.
// Wave w takes the z-plane w of the box, its 32 queries in y-major order.
//
//  1. Logits on the vector units, as in k_local_pair: lanes 2n, 2n+1 serve
//     query n (one channel half each); RoPE enters through the relative
//     angles -1, 0, +1 of each axis, v_dot2 on bf16 pairs, the halves meet
//     through a DPP swap, and the softmax is exact in canonical offset order
//     (maximum first). The bf16 weights, packed as triples (dx = -1, 0, +1)
//     of each (dz, dy), then move to the matrix core's lane layout (lanes n,
//     n + 32 for query n). The denominator sums the same bf16 weights.
//  2. Values are staged row-major, as keys are, into the same LDS buffer once
//     the logits are done.
//  3. O^T (two 32-row tiles of channels x 32 queries) += V^T * P^T with
//     v_mfma_f32_32x32x16_bf16 (channels 48..63 of the second tile read the
//     next row's first channels and are dropped), over the 3 planes x 4
//     blocks of 16 sites a plane of queries can see
//     (site kappa = y*10 + x of a halo plane; 60 sites padded to 64, the
//     padding sites carrying weight 0). The A operand -- one channel of 8
//     consecutive sites per lane -- comes straight from the row-major values
//     through the LDS transpose load ds_read_b64_tr_b16: within a 16-lane
//     group, lane 4q + c receives element c of the 8-byte rows addressed by
//     lanes q, q+4, q+8, q+12, so lane q + 4e addresses site kappa0 + e at
//     the channel quad of lane group q. The B operand holds the query's
//     weights for the 8 sites kappa0 + 8*half ..: its neighbours there form
//     at most one run of three consecutive sites (dx = -1, 0, +1) per block,
//     since the runs of one plane are ten sites apart, so the lane places one
//     bf16 triple at a slot offset with byte permutes and zeros elsewhere.
// The weights are rounded to bf16 for the product and summed in fp32, as in
// the vector kernel; every sum's order is fixed by the query's position in
// its coordinate box, so a repack of the tokens permutes the output bit for
// bit.
#include "launch.hpp"

namespace pk {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s *lds_v4s;
}  // namespace

template <bool MIX>
__global__ __launch_bounds__(256, 1) void k_local_tr48(
    Geo g, const void *geom, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const bf16 *gate, const bf16 *oglob, bf16 *out, int ntz, int nty,
    int ntx) {
  constexpr int D = 48, DA = 16;
  constexpr int TZ = 4, TY = 4, TX = 8;
  constexpr int HZ = TZ + 2, HY = TY + 2, HX = TX + 2, NPL = HY * HX, NH = HZ * NPL;  // 60, 360
  constexpr int NT = 256;
  constexpr int CPS = D / 8;               // 16-byte chunks per row
  constexpr int NCK = NH * CPS;            // 2160 chunks per staged tensor
  constexpr int RS = (NCK + NT - 1) / NT;  // 9 staging rounds
  // One buffer: key rows [site][48] for the logits, then value rows, same
  // layout. Rows past the halo (padding of the last round) hold copies of
  // real rows, so every operand read stays in the buffer and finite.
  __shared__ __attribute__((aligned(16))) bf16 sbuf[RS * NT * 8];
  __shared__ int sSlot[NH];
  __shared__ float sBias[NH];  // 0 for a site with a token, -inf for one without
  // the furthest operand read: padding site 63 of the last plane, channel 63
  static_assert(((HZ - 1) * NPL + 64) * D + (64 - D) <= RS * NT * 8,
                "padding sites and channels stay in the buffer");

  const BoxWork wk = box_work(xcd_remap(blockIdx.x, gridDim.x), g.H, ntz, nty, ntx);
  const int h = wk.h, b = wk.b;
  const int z0 = wk.tz * TZ, y0 = wk.ty * TY, x0 = wk.tx * TX;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int64_t bN = (int64_t)b * g.N;
  // this (batch, KV head)'s rows: token j's row starts j * rstride bytes in
  const int64_t kvbase = (bN * g.Hkv + h / g.G) * D;
  const char *kb = reinterpret_cast<const char *>(k + kvbase);
  const char *vb = reinterpret_cast<const char *>(v + kvbase);
  const uint32_t rstride = (uint32_t)g.Hkv * D * sizeof(bf16);
  {
    constexpr int RSL = (NH + NT - 1) / NT;
    int sv[RSL];
#pragma unroll
    for (int r = 0; r < RSL; r++) {
      const int hs = min((int)threadIdx.x + r * NT, NH - 1);
      const int hz = hs / NPL, hy = (hs / HX) % HY, hx = hs % HX;
      const int z = z0 - 1 + hz, y = y0 - 1 + hy, x = x0 - 1 + hx;
      const bool on = z >= 0 && y >= 0 && x >= 0 && z < g.Z && y < g.Y && x < g.X;
      const int j = slot_get(g, slot, on ? site_of(g, z, y, x) : 0);
      sv[r] = on ? j : -1;
    }
#pragma unroll
    for (int r = 0; r < RSL; r++)
      if ((int)threadIdx.x + r * NT < NH) {
        sSlot[threadIdx.x + r * NT] = sv[r];
        sBias[threadIdx.x + r * NT] = sv[r] >= 0 ? 0.f : -INFINITY;
      }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int tz = threadIdx.x >> 6;  // the wave's plane of queries
  // Logits layout: lanes 2n, 2n + 1 serve query n (channel halves hh).
  // Product layout: lanes n, n + 32 serve query n (site halves hi).
  const int qn = lane >> 1, hh = lane & 1;
  const int qsL = ((tz + 1) * HY + (qn >> 3) + 1) * HX + (qn & 7) + 1;
  const int iL = sSlot[qsL];
  const int hi = lane >> 5, ql = lane & 31;
  const int ty = ql >> 3, tx = ql & 7;
  const int i = sSlot[((tz + 1) * HY + (ty + 1)) * HX + (tx + 1)];
  const int wbase = __builtin_amdgcn_readfirstlane(threadIdx.x & ~63);

  // The loads the logits wait for go out together: key chunks straight into
  // LDS, value chunks into registers, this lane's query slices and the
  // one-step (cos, sin) of its planes. A site off the grid reads token 0
  // (only finiteness matters: its weight is exactly 0).
  bf16x8 vraw[RS];
#pragma unroll
  for (int r = 0; r < RS; r++) {
    const int e = min((int)threadIdx.x + r * NT, NCK - 1);
    const int hs = e / CPS, ch = e % CPS;
    const uint64_t off = (uint64_t)(uint32_t)max(sSlot[hs], 0) * rstride + (uint32_t)ch * 16u;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(kb + off),
                                     (lds_ptr)&sbuf[(wbase + r * NT) * 8], 16, 0, 0);
    vraw[r] = *reinterpret_cast<const bf16x8 *>(vb + off);
  }
  const int64_t row = ((bN + max(i, 0)) * g.H + h) * D;
  const int64_t rowL = ((bN + max(iL, 0)) * g.H + h) * D;
  bf16x8 qraw[3];
#pragma unroll
  for (int a = 0; a < 3; a++) qraw[a] = *reinterpret_cast<const bf16x8 *>(q + rowL + a * DA + 8 * hh);
  float2 cs1[3][4];
#pragma unroll
  for (int a = 0; a < 3; a++) {
    const int dim = a == 0 ? g.Z : (a == 1 ? g.Y : g.X);
#pragma unroll
    for (int u = 0; u < 4; u++) cs1[a][u] = rope_cs(tab, g, a, min(1, dim - 1), 4 * hh + u);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // The fused mix's O_glob slices and gate go out only now: issued with the
  // gathers above they delay them, and they are not needed before the end.
  // They hold this lane's output channels once the halves have traded
  // pieces (below): 16*m + 8*hi .. +7 for m = 0, 1, 2.
  bf16x8 ograw[3];
  float gl = 0.f;
  if constexpr (MIX) {
#pragma unroll
    for (int m = 0; m < 3; m++)
      ograw[m] = *reinterpret_cast<const bf16x8 *>(oglob + row + 16 * m + 8 * hi);
    gl = (float)gate[(bN + max(i, 0)) * g.H + h];
  }
  const float qscale = g.scale * kLog2e;

  // query slices, scaled, rotated by the relative angles -1, 0, +1 of each axis
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

  // logits (log2 units) in canonical offset order k = (dz+1)*9 + (dy+1)*3 + dx+1.
  // The key slices of neighbour k + PF are read while neighbour k is summed
  // (each step its own scheduling region), so LDS latency hides under the
  // dot products instead of stalling every neighbour.
  constexpr int PF = 2;
  float lg[27];
  float mx = -INFINITY;
  bf16x8 kbuf[PF + 1][3];
  float bbuf[PF + 1];
  auto kload = [&](int kk, bf16x8 *dst, float &bias) {
    const int hs = qsL + (kk / 9 - 1) * NPL + ((kk / 3) % 3 - 1) * HX + kk % 3 - 1;
#pragma unroll
    for (int a = 0; a < 3; a++) dst[a] = *reinterpret_cast<const bf16x8 *>(sbuf + hs * D + a * DA + 8 * hh);
    bias = sBias[hs];
  };
#pragma unroll
  for (int kk = 0; kk < PF; kk++) kload(kk, kbuf[kk], bbuf[kk]);
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    __builtin_amdgcn_sched_barrier(0);
    if (kk + PF < 27) kload(kk + PF, kbuf[(kk + PF) % (PF + 1)], bbuf[(kk + PF) % (PF + 1)]);
    const int dd[3] = {kk / 9 - 1, (kk / 3) % 3 - 1, kk % 3 - 1};
    const bf16x8 *kr = kbuf[kk % (PF + 1)];
    float acc = 0.f;
#pragma unroll
    for (int a = 0; a < 3; a++)
#pragma unroll
      for (int u = 0; u < 4; u++) {
        bf16x2 kp;
        kp[0] = kr[a][2 * u];
        kp[1] = kr[a][2 * u + 1];
        acc = __builtin_amdgcn_fdot2_f32_bf16(qv[a][dd[a] + 1][u], kp, acc, false);
      }
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc),
                                                                  0xB1, 0xf, 0xf,
                                                                  true));  // quad_perm 1,0,3,2
    lg[kk] = acc + bbuf[kk % (PF + 1)];
    mx = fmaxf(mx, lg[kk]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the keys are no longer read: the buffer takes the values, row-major
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RS; r++)
    *reinterpret_cast<bf16x8 *>(&sbuf[((int)threadIdx.x + r * NT) * 8]) = vraw[r];
  // bf16 weight triples (dx = -1, 0, +1) of each (dz, dy), packed as the
  // words (p-, p0) and (p+, 0); the denominator sums the same bf16 weights
  uint32_t tev[9][2];
  float den = 0.f;
  bf16x2 ones;
  ones[0] = ones[1] = (bf16)1.0f;
#pragma unroll
  for (int r9 = 0; r9 < 9; r9++) {
    bf16x2 t0, t1;
    t0[0] = (bf16)__builtin_amdgcn_exp2f(lg[3 * r9] - mx);  // 0 for an invalid neighbour
    t0[1] = (bf16)__builtin_amdgcn_exp2f(lg[3 * r9 + 1] - mx);
    t1[0] = (bf16)__builtin_amdgcn_exp2f(lg[3 * r9 + 2] - mx);
    t1[1] = (bf16)0.0f;
    den = __builtin_amdgcn_fdot2_f32_bf16(t0, ones, den, false);  // exact products
    den = __builtin_amdgcn_fdot2_f32_bf16(t1, ones, den, false);
    tev[r9][0] = __builtin_bit_cast(uint32_t, t0);
    tev[r9][1] = __builtin_bit_cast(uint32_t, t1);
  }
  // into the product layout: query n's words come from lane 2n
#pragma unroll
  for (int r9 = 0; r9 < 9; r9++)
#pragma unroll
    for (int j = 0; j < 2; j++) tev[r9][j] = (uint32_t)__shfl((int)tev[r9][j], 2 * ql);
  den = __shfl(den, 2 * ql);
  __syncthreads();

  // Where this lane's weights sit in block kb4 (0..3) of a plane: its window
  // is sites kappa0 = 16*kb4 + 8*hi .. +7; the run of neighbour row dy starts
  // at s_dy = (ty + 1 + dy)*10 + tx, and at most one run meets the window, at
  // slot offset o = s_dy - kappa0 in [-2, 7]. The window's four words are
  // byte permutes of that run's even-packed pair (p-, p0), (p+, 0): for even
  // o = 2m, words m and m+1 are the pair itself; for odd o = 2m + 1 they are
  // (0, p-) and (p0, p+); every other word is zero (selector byte 0x0C).
  f32x16 acc2[2];
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int j = 0; j < 16; j++) acc2[t][j] = 0.f;
  // A operand addresses: lane r = l % 16 of its group serves as row q + 4e
  // (q = r % 4, e = r / 4): site kappa0 + e (second read: + 4) at channels
  // 32t + 16*grp + 4q .. +3 of its plane; rows of plane dzi start
  // (tz + dzi) * 60 sites into the buffer
  const int grp = (lane >> 4) & 1, rq = lane & 3, re = (lane >> 2) & 3;
  const int abase = (tz * NPL + re) * D + 16 * grp + 4 * rq;  // elements
#pragma unroll
  for (int kb4 = 0; kb4 < 4; kb4++) {
    const int k0 = 16 * kb4 + 8 * hi;
    const int sm = ty * 10 + tx;  // s_{-1}
    // run di = dy + 1 meets the window iff 10*di lies in [k0 - sm - 2, k0 - sm + 7],
    // ten consecutive integers: exactly one multiple of ten
    const int rel = k0 - sm + 7;
    const int di = rel >= 0 ? rel / 10 : -1;
    const bool ok = di >= 0 && di <= 2;
    const int o = sm + 10 * di - k0;
    const int m = ok ? (o >> 1) : -8;  // arithmetic shift: floor
    const bool odd = (o & 1) != 0;
    const uint32_t s0 = odd ? 0x01000C0Cu : 0x03020100u, s1 = odd ? 0x05040302u : 0x07060504u;
    uint32_t sel[4];
#pragma unroll
    for (int jd = 0; jd < 4; jd++) sel[jd] = jd == m ? s0 : (jd == m + 1 ? s1 : 0x0C0C0C0Cu);
#pragma unroll
    for (int dzi = 0; dzi < 3; dzi++) {
      // the even-packed triple of run di of plane dzi (any, when no run meets)
      const uint32_t x0 = di == 0 ? tev[3 * dzi][0] : (di == 1 ? tev[3 * dzi + 1][0] : tev[3 * dzi + 2][0]);
      const uint32_t x1 = di == 0 ? tev[3 * dzi][1] : (di == 1 ? tev[3 * dzi + 1][1] : tev[3 * dzi + 2][1]);
      uint32_t bw[4];
#pragma unroll
      for (int jd = 0; jd < 4; jd++) bw[jd] = __builtin_amdgcn_perm(x1, x0, sel[jd]);
      bf16x8 bop;
      __builtin_memcpy(&bop, bw, 16);
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int ad = abase + (dzi * NPL + k0) * D + 32 * t;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(sbuf + ad));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(sbuf + ad + 4 * D));
        bf16x8 aop;
        __builtin_memcpy(&aop, &lo, 8);
        __builtin_memcpy(reinterpret_cast<char *>(&aop) + 8, &hi4, 8);
        acc2[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, acc2[t], 0, 0, 0);
      }
    }
  }
  // The product layout gives lane (n, hi) channels 8*jj + 4*hi .. +3 of
  // query n (tile jj / 4, registers 4*(jj % 4) ..). The two halves trade
  // pieces so that each lane holds 8 consecutive channels 16*m + 8*hi .. +7:
  // whole 16-byte pieces of the row for the O_glob reads and the stores.
  // v_permlane32_swap exchanges lanes 32..63 of its first operand with
  // lanes 0..31 of its second: with (piece 2m, piece 2m + 1) as operands the
  // first result is channels 16m + 8hi .. +3 and the second the 4 after them.
  const float inv = 1.0f / den;
  float oc[3][8];
#pragma unroll
  for (int m = 0; m < 3; m++)
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const float e0 = acc2[(2 * m) / 4][4 * ((2 * m) % 4) + u];          // piece 2m
      const float e1 = acc2[(2 * m + 1) / 4][4 * ((2 * m + 1) % 4) + u];  // piece 2m + 1
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, e0),
                                                       __builtin_bit_cast(uint32_t, e1), false,
                                                       false);
      oc[m][u] = __builtin_bit_cast(float, (uint32_t)sw[0]);
      oc[m][4 + u] = __builtin_bit_cast(float, (uint32_t)sw[1]);
    }
  if (i < 0) return;
  // O = (1 - g) * acc / den + g * O_glob, with (1 - g) / den taken once
  float gg = 0.f, sl = inv;
  if constexpr (MIX) {
    gg = 1.0f / (1.0f + expf(-gl));
    sl = (1.0f - gg) * inv;
  }
#pragma unroll
  for (int m = 0; m < 3; m++) {
    bf16x8 r;
#pragma unroll
    for (int u = 0; u < 8; u++) {
      if constexpr (MIX)
        r[u] = (bf16)fmaf(oc[m][u], sl, gg * (float)ograw[m][u]);
      else
        r[u] = (bf16)(oc[m][u] * sl);
    }
    *reinterpret_cast<bf16x8 *>(out + row + 16 * m + 8 * hi) = r;
  }
}

hipError_t launch_local_tr48(const Geo &g, const void *geom, const void *q, const void *k,
                             const void *v, const void *gate, const void *og, void *out,
                             hipStream_t s) {
  const int ntz = (g.Z + 3) / 4, nty = (g.Y + 3) / 4, ntx = (g.X + 7) / 8;
  const int64_t nwg = (int64_t)g.B * ntz * nty * ntx * g.H;
  const bool mix = gate != nullptr;
  hipLaunchKernelGGL(mix ? k_local_tr48<true> : k_local_tr48<false>, dim3((unsigned)nwg),
                     dim3(256), 0, s, g, geom, static_cast<const bf16 *>(q),
                     static_cast<const bf16 *>(k), static_cast<const bf16 *>(v),
                     static_cast<const bf16 *>(gate), static_cast<const bf16 *>(og),
                     static_cast<bf16 *>(out), ntz, nty, ntx);
  return hipGetLastError();
}

}  // namespace pk
