// Global branch of the backward on bf16 matrix cores (Geometry Matters in
// Packed 3D Attention: the backward of the query-to-summary attention,
// project page Ch. 3, Contract 2; paper summary §3.4, §3.5). With
// t_im = <q~_i, k_sum_m> * s * log2(e) and the forward's log-sum-exp lse_i:
//   P = exp2(t - lse), dP = dO_glob * v_sum^T, dT = P (dP - Delta),
//   dq~   = s    * dT  * k_sum            (query side)
//   dk_sum = s   * dT^T * q~,  dv_sum = P^T * dO_glob   (summary side)
// Three dense contractions per (query, summary) pair on the query side and
// four on the summary side; like the forward, no token x summary matrix is
// ever stored.
//
// Both sides use the forward's register trick: a 32x32 score block comes out
// of v_mfma_f32_32x32x16_bf16 with each lane holding 16 values of one column,
// and placing the contraction rows in bit-2/3-swapped order makes those 16
// values exactly the next product's operand fragment (k index
// 16*c2 + 8*hi + e for register 8*c2 + e of half-wave hi).
//
//   k_bwd_prep_mfma   per (batch, query head, grid site): bf16 q~ s log2(e)
//                     and dO_glob = g dO (rounded as the forward rounds q~),
//                     in 32-row blocks and 8-row transposed blocks, with the
//                     saved lse and Delta = <dO_glob, O_glob>, in grid-site
//                     (raster) order -- the order every reduction runs in
//   k_bwd_relayout    v_sum in the key-summary layout and k_sum in the
//                     value-summary layout, the operand shapes the
//                     contractions above need
//   k_bwd_gq_mfma     query side: a wave owns 32 query sites and streams the
//                     summaries through LDS
//   k_bwd_gk_mfma     summary side: a wave owns 32 summaries and streams the
//                     query sites of one split of the site range through LDS
//   k_bwd_split_sum   the splits' partial sums, added in split order
#include <type_traits>

#include "launch.hpp"

namespace pk {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSiteAlign = 256;  // query sites padded to whole query tiles of every kernel

__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
}  // namespace

// ---------------------------------------------------------------------------
// Position p of (b, h) is grid site p (raster order), p < Np = 256*ceil(N/256):
//   qn [B*H, Np/32, D/8, 32, 8]  q~ s log2(e): row p%32 of 32-row block p/32
//   qt [B*H, Np/8, D, 8]         the same, channel-major: 8 sites per chunk
//   dn, dt                       dO_glob, likewise
//   lse_p, dl_p [B*H, Np]        saved lse (+inf where no token: P = 0), Delta
//   tok [B, Np]                  token at the site (-1: none)
template <int D>
__global__ __launch_bounds__(256) void k_bwd_prep_mfma(
    Geo g, const void *geom, const bf16 *__restrict__ q, const bf16 *__restrict__ gate,
    const bf16 *__restrict__ dout, const bf16 *__restrict__ oglob, const float *__restrict__ lse,
    bf16 *qn, bf16 *qt, bf16 *dn, bf16 *dt, float *lse_p, float *dl_p, int32_t *tok, int Np) {
  constexpr int DA = D / 3, NCH = D / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // ((b*H + h) * Np + p)
  if (t >= (int64_t)g.B * g.H * Np) return;
  const int p = (int)(t % Np);
  const int64_t bh = t / Np;
  const int h = (int)(bh % g.H), b = (int)(bh / g.H);
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int i = p < g.N ? slot[p] : -1;
  if (h == 0) tok[(int64_t)b * Np + p] = i;
  const int c3[3] = {p / (g.Y * g.X), (p / g.X) % g.Y, p % g.X};
  const int64_t row = ((int64_t)b * g.N + max(i, 0)) * g.H + h;
  const float qscale = g.scale * kLog2e;
  const float gg = i >= 0 ? 1.0f / (1.0f + expf(-(float)gate[row])) : 0.f;
  float dl = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    bf16x8 qv, dv;
    if (i >= 0) {
      const bf16x8 raw = *reinterpret_cast<const bf16x8 *>(q + row * D + 8 * c);
      const bf16x8 draw = *reinterpret_cast<const bf16x8 *>(dout + row * D + 8 * c);
      const bf16x8 oraw = *reinterpret_cast<const bf16x8 *>(oglob + row * D + 8 * c);
      const int a = (8 * c) / DA, p0 = ((8 * c) % DA) / 2;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        float x0 = (float)raw[2 * u], x1 = (float)raw[2 * u + 1];
        rotate(x0, x1, rope_cs(tab, g, a, c3[a], p0 + u));
        qv[2 * u] = (bf16)(x0 * qscale);
        qv[2 * u + 1] = (bf16)(x1 * qscale);
      }
#pragma unroll
      for (int e = 0; e < 8; e++) {
        dv[e] = (bf16)(gg * (float)draw[e]);
        dl += (float)dv[e] * (float)oraw[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; e++) qv[e] = dv[e] = (bf16)0.0f;
    }
    const int64_t nb = (((bh * (Np / 32) + p / 32) * NCH + c) * 32 + p % 32) * 8;
    *reinterpret_cast<bf16x8 *>(qn + nb) = qv;
    *reinterpret_cast<bf16x8 *>(dn + nb) = dv;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int64_t tb = ((bh * (Np / 8) + p / 8) * D + 8 * c + e) * 8 + p % 8;
      qt[tb] = qv[e];
      dt[tb] = dv[e];
    }
  }
  lse_p[t] = i >= 0 ? lse[row] : INFINITY;
  dl_p[t] = dl;
}

// v_sum [B*Hkv, Mp/8, D, 8] -> vk [B*Hkv, Mp/32, D/8, 32, 8] and
// k_sum [B*Hkv, Mp/32, D/8, 32, 8] -> kt [B*Hkv, Mp/8, D, 8]
template <int D>
__global__ void k_bwd_relayout(int64_t n, int Mp, const bf16 *__restrict__ ks,
                               const bf16 *__restrict__ vs, bf16 *vk, bf16 *kt) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (bk, m, d)
  if (e >= n) return;
  const int d = (int)(e % D);
  const int m = (int)((e / D) % Mp);
  const int64_t bk = e / ((int64_t)D * Mp);
  const int64_t kso = (((bk * (Mp / 32) + m / 32) * (D / 8) + d / 8) * 32 + m % 32) * 8 + d % 8;
  const int64_t vso = ((bk * (Mp / 8) + m / 8) * D + d) * 8 + m % 8;
  vk[kso] = vs[vso];
  kt[vso] = ks[kso];
}

// ---------------------------------------------------------------------------
// Query side. Workgroup: NW waves, each owning G groups of 32 query sites of
// one (b, h) that share every LDS fragment read; summary tiles of TS (NSUB
// 32-summary sub-tiles) double-buffered in LDS, filled by buffer loads
// straight into LDS (16 bytes per lane, offsets computed once): the loads of
// tile t+1 go out while tile t is used, one barrier per tile. With G = 2 one
// group's vector work runs while the matrix core works on the other's.
template <int D, int TS, int NW, int G>
__global__ __launch_bounds__(64 * NW, G == 1 ? 2 : 1) void k_bwd_gq_mfma(
    Geo g, const bf16 *__restrict__ qn, const bf16 *__restrict__ dn,
    const float *__restrict__ lse_p, const float *__restrict__ dl_p,
    const int32_t *__restrict__ tok, const bf16 *__restrict__ ks, const bf16 *__restrict__ vk,
    const bf16 *__restrict__ kt, float *dqg, int Np, int ntiles) {
  constexpr int KD = D / 16, NCH = D / 8, DT = (D + 31) / 32, NSUB = TS / 32;
  constexpr int NJ8 = TS / 8;
  // chunks per tile: k_sum and vk rows (NCH x TS), kt (NJ8 x D); whole waves
  constexpr int NKC = NCH * TS, NTC = NJ8 * D, NTH = 64 * NW;
  static_assert(NKC % 64 == 0 && NTC % 64 == 0, "tile loads in whole waves");
  constexpr int RK = (NKC + NTH - 1) / NTH, RT = (NTC + NTH - 1) / NTH;
  __shared__ bf16x8 sK0[NKC], sK1[NKC], sV0[NKC], sV1[NKC], sT0[NTC], sT1[NTC];
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = w % ntiles, bh = w / ntiles;
  const int h = bh % g.H, b = bh / g.H;
  const int lane = threadIdx.x & 63, hi = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Mp = (g.M + 31) / 32 * 32, M32 = Mp / 32;
  const int64_t bk = (int64_t)b * g.Hkv + h / g.G;
  // this lane's query site of each group (Np is a multiple of NW * 32 * G)
  int p[G];
  bf16x8 qf[G][KD], df[G][KD];
  float lq[G], dq[G];
  f32x16 acc[G][DT];
#pragma unroll
  for (int gi = 0; gi < G; gi++) {
    p[gi] = tile * (NW * 32 * G) + (wv * G + gi) * 32 + l32;
#pragma unroll
    for (int c = 0; c < KD; c++) {
      const int64_t o =
          ((((int64_t)bh * (Np / 32) + p[gi] / 32) * NCH + 2 * c + hi) * 32 + p[gi] % 32) * 8;
      qf[gi][c] = *reinterpret_cast<const bf16x8 *>(qn + o);
      df[gi][c] = *reinterpret_cast<const bf16x8 *>(dn + o);
    }
    lq[gi] = lse_p[(int64_t)bh * Np + p[gi]];
    dq[gi] = dl_p[(int64_t)bh * Np + p[gi]];
#pragma unroll
    for (int t = 0; t < DT; t++)
#pragma unroll
      for (int j = 0; j < 16; j++) acc[gi][t][j] = 0.f;
  }
  const f32x16 zero16 = {};

  // per-lane parts of the tile offsets: row chunk e = (ch, pos) holds summary
  // 32*(pos/32) + swap23(pos%32) of the tile; kt chunk e = (j8, d)
  int rk_sub[RK], rk_in[RK], rt_j8[RT], rt_d[RT];
#pragma unroll
  for (int r = 0; r < RK; r++) {
    const int e = NTH * r + 64 * wv + lane;
    const int ch = e / TS, pos = e % TS;
    rk_sub[r] = pos / 32;
    rk_in[r] = (ch * 32 + swap23(pos % 32)) * 8;
  }
#pragma unroll
  for (int r = 0; r < RT; r++) {
    const int e = NTH * r + 64 * wv + lane;
    rt_j8[r] = e / D;
    rt_d[r] = e % D;
  }
  // this KV head's k_sum, V-in-key-layout and K-in-value-layout slices
  const __amdgpu_buffer_rsrc_t rks = buffer_rsrc(ks + bk * M32 * (NCH * 256), M32 * NCH * 512);
  const __amdgpu_buffer_rsrc_t rvk = buffer_rsrc(vk + bk * M32 * (NCH * 256), M32 * NCH * 512);
  const __amdgpu_buffer_rsrc_t rkt = buffer_rsrc(kt + bk * 4 * M32 * D * 8, 4 * M32 * D * 16);
  auto issue = [&](int tt, bf16x8 *dK, bf16x8 *dV, bf16x8 *dT) {
#pragma unroll
    for (int r = 0; r < RK; r++) {
      if (NTH * r + 64 * wv < NKC) {  // wave-uniform
        const int m32 = min(tt * NSUB + rk_sub[r], M32 - 1);
        const uint32_t o = (uint32_t)(m32 * (NCH * 256) + rk_in[r]) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, (lds_ptr)&dK[NTH * r + 64 * wv], 16, o, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rvk, (lds_ptr)&dV[NTH * r + 64 * wv], 16, o, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < RT; r++) {
      if (NTH * r + 64 * wv < NTC) {
        const int g8 = min(tt * NJ8 + rt_j8[r], 4 * M32 - 1);
        const uint32_t o = (uint32_t)(g8 * D + rt_d[r]) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rkt, (lds_ptr)&dT[NTH * r + 64 * wv], 16, o, 0, 0, 0);
      }
    }
  };
  // one 32-summary sub-tile for every group; MASK zeroes the summaries at or
  // past M
  auto sub_step = [&](const bf16x8 *K, const bf16x8 *V, const bf16x8 *T, int sub, int mbase,
                      auto mask) {
    f32x16 s[G], dp[G];
#pragma unroll
    for (int c = 0; c < KD; c++) {
      const bf16x8 kf = K[(2 * c + hi) * TS + 32 * sub + l32];
      const bf16x8 vf = V[(2 * c + hi) * TS + 32 * sub + l32];
#pragma unroll
      for (int gi = 0; gi < G; gi++) {
        s[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[gi][c], c == 0 ? zero16 : s[gi], 0, 0, 0);
        dp[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[gi][c], c == 0 ? zero16 : dp[gi], 0, 0, 0);
      }
    }
#pragma unroll
    for (int gi = 0; gi < G; gi++) {
      // register j <-> summary mbase + 16*(j/8) + 8*hi + j%8
      bf16x8 tf[2];
#pragma unroll
      for (int j = 0; j < 16; j++) {
        float t = __builtin_amdgcn_exp2f(s[gi][j] - lq[gi]) * (dp[gi][j] - dq[gi]);
        if constexpr (decltype(mask)::value)
          t = (mbase + 16 * (j >> 3) + 8 * hi + (j & 7) < g.M) ? t : 0.f;
        tf[j >> 3][j & 7] = (bf16)t;
      }
#pragma unroll
      for (int t = 0; t < DT; t++) {
        const int d = min(32 * t + l32, D - 1);
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++) {
          const bf16x8 kf2 = T[(4 * sub + 2 * c2 + hi) * D + d];
          acc[gi][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf2, tf[c2], acc[gi][t], 0, 0, 0);
        }
      }
    }
  };
  const int ntile = (M32 + NSUB - 1) / NSUB;
  issue(0, sK0, sV0, sT0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int tt = 0; tt < ntile; tt++) {
    const bool odd = tt & 1;
    if (tt + 1 < ntile) {
      if (odd) issue(tt + 1, sK0, sV0, sT0);
      else issue(tt + 1, sK1, sV1, sT1);
    }
    const bf16x8 *K = odd ? sK1 : sK0, *V = odd ? sV1 : sV0, *T = odd ? sT1 : sT0;
    if ((tt + 1) * TS <= g.M && G == 1) {
      // a whole tile below M: the score products of every sub-tile first, so
      // that each sub-tile's vector work overlaps the matrix core's work on
      // the next sub-tile (and on the previous one's accumulation)
      f32x16 s[NSUB], dp[NSUB];
#pragma unroll
      for (int sub = 0; sub < NSUB; sub++)
#pragma unroll
        for (int c = 0; c < KD; c++) {
          const bf16x8 kf = K[(2 * c + hi) * TS + 32 * sub + l32];
          const bf16x8 vf = V[(2 * c + hi) * TS + 32 * sub + l32];
          s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[0][c], c == 0 ? zero16 : s[sub], 0, 0, 0);
          dp[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[0][c], c == 0 ? zero16 : dp[sub], 0, 0, 0);
        }
#pragma unroll
      for (int sub = 0; sub < NSUB; sub++) {
        bf16x8 tf[2];
#pragma unroll
        for (int j = 0; j < 16; j++)
          tf[j >> 3][j & 7] =
              (bf16)(__builtin_amdgcn_exp2f(s[sub][j] - lq[0]) * (dp[sub][j] - dq[0]));
#pragma unroll
        for (int t = 0; t < DT; t++) {
          const int d = min(32 * t + l32, D - 1);
#pragma unroll
          for (int c2 = 0; c2 < 2; c2++) {
            const bf16x8 kf = T[(4 * sub + 2 * c2 + hi) * D + d];
            acc[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, tf[c2], acc[0][t], 0, 0, 0);
          }
        }
      }
    } else if ((tt + 1) * TS <= g.M) {
#pragma unroll
      for (int sub = 0; sub < NSUB; sub++) sub_step(K, V, T, sub, 0, std::false_type{});
    } else {
#pragma unroll
      for (int sub = 0; sub < NSUB; sub++) {
        const int mbase = tt * TS + 32 * sub;
        if (mbase >= Mp) break;  // uniform: the last tile may be partial
        if (mbase + 32 <= g.M)
          sub_step(K, V, T, sub, mbase, std::false_type{});
        else
          sub_step(K, V, T, sub, mbase, std::true_type{});
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tile have landed
    __syncthreads();
  }
  // lane: query site p (column l32), rows d = 32t + 8jj + 4hi + u
#pragma unroll
  for (int gi = 0; gi < G; gi++) {
    const int i = p[gi] < g.N ? tok[(int64_t)b * Np + p[gi]] : -1;
    if (i < 0) continue;
    float *orow = dqg + (((int64_t)b * g.N + i) * g.H + h) * D;
#pragma unroll
    for (int t = 0; t < DT; t++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int d = 32 * t + 8 * jj + 4 * hi;
        if (d < D) {
          f32x4 o4;
#pragma unroll
          for (int u = 0; u < 4; u++) o4[u] = g.scale * acc[gi][t][4 * jj + u];
          *reinterpret_cast<f32x4 *>(orow + d) = o4;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Summary side. Workgroup: 4 waves x 32 summaries of one (b, hk), one split
// of the query sites of every head of the group; query tiles of TQ sites
// double-buffered in LDS by buffer loads straight into LDS (Np is a multiple
// of 256, so every tile is whole). Writes the split's partial sums.
template <int D, int TQ, int NW>
__global__ __launch_bounds__(64 * NW, 2) void k_bwd_gk_mfma(
    Geo g, const bf16 *__restrict__ qn, const bf16 *__restrict__ qt, const bf16 *__restrict__ dn,
    const bf16 *__restrict__ dt, const float *__restrict__ lse_p, const float *__restrict__ dl_p,
    const bf16 *__restrict__ ks, const bf16 *__restrict__ vk, float *dks_part, float *dvs_part,
    int Np, int mtiles, int nsplit) {
  constexpr int KD = D / 16, NCH = D / 8, DT = (D + 31) / 32, NSUB = TQ / 32, NJ8 = TQ / 8;
  constexpr int NNC = NCH * TQ, NTC = NJ8 * D, NTH = 64 * NW;  // chunks per tile
  static_assert(NNC % 64 == 0 && NTC % 64 == 0 && TQ <= 64, "tile loads in whole waves");
  constexpr int RN = (NNC + NTH - 1) / NTH, RTT = (NTC + NTH - 1) / NTH;
  __shared__ bf16x8 sQ0[NNC], sQ1[NNC], sD0[NNC], sD1[NNC];
  __shared__ bf16x8 sQT0[NTC], sQT1[NTC], sDT0[NTC], sDT1[NTC];
  __shared__ __attribute__((aligned(16))) float sL0[64], sL1[64], sDl0[64], sDl1[64];
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int split = w % nsplit, mt = (w / nsplit) % mtiles, bk = w / (nsplit * mtiles);
  const int b = bk / g.Hkv, hk = bk % g.Hkv;
  const int lane = threadIdx.x & 63, hi = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Mp = (g.M + 31) / 32 * 32;
  const int m32 = min(mt * NW + wv, Mp / 32 - 1);  // this wave's 32 summaries
  const bool wave_live = mt * NW + wv < Mp / 32;
  bf16x8 kb[KD], vb[KD];
#pragma unroll
  for (int c = 0; c < KD; c++) {
    const int64_t o = ((((int64_t)bk * (Mp / 32) + m32) * NCH + 2 * c + hi) * 32 + l32) * 8;
    kb[c] = *reinterpret_cast<const bf16x8 *>(ks + o);
    vb[c] = *reinterpret_cast<const bf16x8 *>(vk + o);
  }
  f32x16 aK[DT], aV[DT];
#pragma unroll
  for (int t = 0; t < DT; t++)
#pragma unroll
    for (int j = 0; j < 16; j++) aK[t][j] = aV[t][j] = 0.f;
  const f32x16 zero16 = {};

  const int nqt = Np / TQ;
  const int per = (nqt + nsplit - 1) / nsplit;
  const int qt0 = split * per, qt1 = min(nqt, qt0 + per);
  const int nq = max(qt1 - qt0, 0);
  const int ntile = nq * g.G;  // (head of the group, query tile) pairs

  int rn_sub[RN], rn_in[RN], rt_j8[RTT], rt_d[RTT];
#pragma unroll
  for (int r = 0; r < RN; r++) {
    const int e = NTH * r + 64 * wv + lane;
    const int ch = e / TQ, pos = e % TQ;
    rn_sub[r] = pos / 32;
    rn_in[r] = (ch * 32 + swap23(pos % 32)) * 8;
  }
#pragma unroll
  for (int r = 0; r < RTT; r++) {
    const int e = NTH * r + 64 * wv + lane;
    rt_j8[r] = e / D;
    rt_d[r] = e % D;
  }
  auto issue = [&](int it, bf16x8 *dQ, bf16x8 *dD, bf16x8 *dQT, bf16x8 *dDT, float *dL,
                   float *dDl) {
    const int h = hk * g.G + it / nq, qtile = qt0 + it % nq;
    const int64_t bh = (int64_t)b * g.H + h;
    // this head's slices: both query layouts are Np * D elements per head
    const int32_t bytes = Np * D * 2;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(qn + bh * Np * D, bytes);
    const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(dn + bh * Np * D, bytes);
    const __amdgpu_buffer_rsrc_t rqt = buffer_rsrc(qt + bh * Np * D, bytes);
    const __amdgpu_buffer_rsrc_t rdt = buffer_rsrc(dt + bh * Np * D, bytes);
#pragma unroll
    for (int r = 0; r < RN; r++) {
      if (NTH * r + 64 * wv < NNC) {
        const uint32_t o = (uint32_t)((qtile * NSUB + rn_sub[r]) * (NCH * 256) + rn_in[r]) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_ptr)&dQ[NTH * r + 64 * wv], 16, o, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_ptr)&dD[NTH * r + 64 * wv], 16, o, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < RTT; r++) {
      if (NTH * r + 64 * wv < NTC) {
        const uint32_t o = (uint32_t)((qtile * NJ8 + rt_j8[r]) * D + rt_d[r]) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rqt, (lds_ptr)&dQT[NTH * r + 64 * wv], 16, o, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rdt, (lds_ptr)&dDT[NTH * r + 64 * wv], 16, o, 0, 0, 0);
      }
    }
    // per-site statistics: wave 0 the log-sum-exp, wave 1 Delta (4 bytes a lane)
    if (wv < 2) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc((wv == 0 ? lse_p : dl_p) + bh * Np, Np * 4);
      const uint32_t o = (uint32_t)(qtile * TQ + min(lane, TQ - 1)) * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(wv == 0 ? dL : dDl), 4, o, 0, 0, 0);
    }
  };
  if (ntile > 0) issue(0, sQ0, sD0, sQT0, sDT0, sL0, sDl0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntile; it++) {
    const bool odd = it & 1;
    if (it + 1 < ntile) {
      if (odd) issue(it + 1, sQ0, sD0, sQT0, sDT0, sL0, sDl0);
      else issue(it + 1, sQ1, sD1, sQT1, sDT1, sL1, sDl1);
    }
    const bf16x8 *Q = odd ? sQ1 : sQ0, *Dd = odd ? sD1 : sD0;
    const bf16x8 *QT = odd ? sQT1 : sQT0, *DTt = odd ? sDT1 : sDT0;
    const float *L = odd ? sL1 : sL0, *Dl = odd ? sDl1 : sDl0;
    // the score products of every sub-tile of the tile first, so that each
    // sub-tile's vector work runs while the matrix core still works on the
    // next one's products (and on the previous one's accumulation)
    // C[query rows][summary columns]: row r holds query site swap23(r)
    f32x16 s[NSUB], dp[NSUB];
#pragma unroll
    for (int sub = 0; sub < NSUB; sub++) {
#pragma unroll
      for (int c = 0; c < KD; c++) {
        const bf16x8 qa = Q[(2 * c + hi) * TQ + 32 * sub + l32];
        const bf16x8 da = Dd[(2 * c + hi) * TQ + 32 * sub + l32];
        s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb[c], c == 0 ? zero16 : s[sub], 0, 0, 0);
        dp[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vb[c], c == 0 ? zero16 : dp[sub], 0, 0, 0);
      }
    }
#pragma unroll
    for (int sub = 0; sub < NSUB; sub++) {
      // register 8*c2 + e of half hi <-> site 32*sub + 16*c2 + 8*hi + e
      bf16x8 pa[2], ta[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++) {
        const int q0 = 32 * sub + 16 * c2 + 8 * hi;
        const f32x4 l0 = *reinterpret_cast<const f32x4 *>(L + q0);
        const f32x4 l1 = *reinterpret_cast<const f32x4 *>(L + q0 + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4 *>(Dl + q0);
        const f32x4 d1 = *reinterpret_cast<const f32x4 *>(Dl + q0 + 4);
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const float le = e < 4 ? l0[e] : l1[e - 4], de = e < 4 ? d0[e] : d1[e - 4];
          const float pr = __builtin_amdgcn_exp2f(s[sub][8 * c2 + e] - le);
          pa[c2][e] = (bf16)pr;
          ta[c2][e] = (bf16)(pr * (dp[sub][8 * c2 + e] - de));
        }
      }
#pragma unroll
      for (int t = 0; t < DT; t++) {
        const int d = min(32 * t + l32, D - 1);
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++) {
          const int j8 = 4 * sub + 2 * c2 + hi;
          const bf16x8 qb = QT[j8 * D + d];
          const bf16x8 db = DTt[j8 * D + d];
          aK[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[c2], qb, aK[t], 0, 0, 0);
          aV[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[c2], db, aV[t], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (!wave_live) return;
  // lane: channel column 32t + l32, rows = summaries 8jj + 4hi + u of the group
  const int64_t base = (((int64_t)split * g.B * g.Hkv + bk) * g.M) * D;
#pragma unroll
  for (int t = 0; t < DT; t++) {
    const int d = 32 * t + l32;
    if (d >= D) continue;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int m = m32 * 32 + (j >> 2) * 8 + hi * 4 + (j & 3);
      if (m < g.M) {
        dks_part[base + (int64_t)m * D + d] = kLn2 * aK[t][j];  // s / (s log2 e)
        dvs_part[base + (int64_t)m * D + d] = aV[t][j];
      }
    }
  }
}

__global__ void k_bwd_split_sum(int64_t n, int nsplit, const float *__restrict__ part, float *out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s = 0.f;
  for (int k = 0; k < nsplit; k++) s += part[k * n + e];
  out[e] = s;
}

// ---------------------------------------------------------------------------
namespace {
template <int D, int TS, int TQ, int NWQ, int GQ, int NWK>
hipError_t run_bwd_global_mfma(const Geo &g, const BwdArgs &a, const BwdMfmaArgs &m,
                               hipStream_t s) {
  const int Np = (g.N + kSiteAlign - 1) / kSiteAlign * kSiteAlign, Mp = (g.M + 31) / 32 * 32;
  {
    const int64_t n = (int64_t)g.B * g.H * Np;
    hipLaunchKernelGGL((k_bwd_prep_mfma<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g,
                       a.geom, static_cast<const bf16 *>(a.q), static_cast<const bf16 *>(a.gate),
                       static_cast<const bf16 *>(a.dout), static_cast<const bf16 *>(a.oglob),
                       a.lse_g, m.qn, m.qt, m.dn, m.dt, m.lse_p, m.dl_p, m.tok, Np);
    if (hipError_t e = hipGetLastError()) return e;
  }
  {
    const int64_t n = (int64_t)g.B * g.Hkv * Mp * D;
    hipLaunchKernelGGL((k_bwd_relayout<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n,
                       Mp, static_cast<const bf16 *>(a.ks), static_cast<const bf16 *>(a.vs), m.vk,
                       m.kt);
    if (hipError_t e = hipGetLastError()) return e;
  }
  {
    const int ntiles = Np / (NWQ * 32 * GQ);
    hipLaunchKernelGGL((k_bwd_gq_mfma<D, TS, NWQ, GQ>), dim3((unsigned)(ntiles * g.B * g.H)), dim3(64 * NWQ), 0, s,
                       g, m.qn, m.dn, m.lse_p, m.dl_p, m.tok, static_cast<const bf16 *>(a.ks), m.vk,
                       m.kt, a.dqg, Np, ntiles);
    if (hipError_t e = hipGetLastError()) return e;
  }
  {
    const int mtiles = (Mp / 32 + NWK - 1) / NWK;
    hipLaunchKernelGGL((k_bwd_gk_mfma<D, TQ, NWK>), dim3((unsigned)(m.nsplit * mtiles * g.B * g.Hkv)),
                       dim3(64 * NWK), 0, s, g, m.qn, m.qt, m.dn, m.dt, m.lse_p, m.dl_p,
                       static_cast<const bf16 *>(a.ks), m.vk, m.dks_part, m.dvs_part, Np, mtiles,
                       m.nsplit);
    if (hipError_t e = hipGetLastError()) return e;
    const int64_t n = (int64_t)g.B * g.Hkv * g.M * D;
    hipLaunchKernelGGL(k_bwd_split_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n,
                       m.nsplit, m.dks_part, a.dks);
    hipLaunchKernelGGL(k_bwd_split_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n,
                       m.nsplit, m.dvs_part, a.dvs);
  }
  return hipGetLastError();
}
}  // namespace

bool bwd_global_mfma_supported(const Geo &g, int dtype) {
  // one head's query slice and one KV head's summaries are addressed with
  // 32-bit byte offsets
  const int64_t Np = ((int64_t)g.N + kSiteAlign - 1) / kSiteAlign * kSiteAlign;
  const int64_t Mp = ((int64_t)g.M + 31) / 32 * 32;
  return dtype == PACK3D_BF16 && g.excl == PACK3D_EXCL_NONE && (g.D == 48 || g.D == 96) &&
         Np * g.D * 2 <= INT32_MAX && Mp * g.D * 2 <= INT32_MAX;
}

hipError_t launch_bwd_global_mfma(const Geo &g, const BwdArgs &a, const BwdMfmaArgs &m,
                                  hipStream_t s) {
  if (g.D == 48) return run_bwd_global_mfma<48, 64, 64, 4, 1, 4>(g, a, m, s);
  return run_bwd_global_mfma<96, 64, 32, 4, 1, 4>(g, a, m, s);
}

}  // namespace pk
