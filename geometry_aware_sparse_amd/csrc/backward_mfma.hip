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
//                     saved lse and Delta = <dO_glob, O_glob>, both negated,
//                     in grid-site (raster) order -- the order every
//                     reduction runs in. The negated values start the
//                     accumulators of the score and dP products, so the
//                     products return t - lse and dP - Delta directly.
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

// bf16 pair w (elements 2w, 2w+1) of v replaced by p, as one 32-bit word
__device__ __forceinline__ bf16x8 set_pair(bf16x8 v, int w, bf16x2 p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 u = __builtin_bit_cast(u32x4, v);
  u[w] = __builtin_bit_cast(uint32_t, p);
  return __builtin_bit_cast(bf16x8, u);
}

// v_permlane16_swap on each 32-bit word of the pair (a[0], a[1]), in place:
// a[0] keeps its lanes 0..15 / 32..47 and takes lanes 0..15 / 32..47 of a[1]
// into its lanes 16..31 / 48..63; a[1] gets the rest (lanes 16..31 / 48..63
// of a[0] in its lanes 0..15 / 32..47, and its own lanes 16..31 / 48..63).
__device__ __forceinline__ void swap_rows16(bf16x8 *a) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_bit_cast(u32x4, a[0]), y = __builtin_bit_cast(u32x4, a[1]);
  u32x4 r0, r1;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    const auto sw = __builtin_amdgcn_permlane16_swap(x[w], y[w], false, false);
    r0[w] = sw[0];
    r1[w] = sw[1];
  }
  a[0] = __builtin_bit_cast(bf16x8, r0);
  a[1] = __builtin_bit_cast(bf16x8, r1);
}
}  // namespace

// ---------------------------------------------------------------------------
// Position p of (b, h) is grid site p (raster order), p < Np = 256*ceil(N/256):
//   qn [B*H, Np/32, D/8, 32, 8]  q~ s log2(e): row p%32 of 32-row block p/32
//   qt [B*H, Np/8, D, 8]         the same, channel-major: 8 sites per chunk
//   dn, dt                       dO_glob, likewise
//   lse_p, dl_p [B*H, Np]        -lse (-inf where no token: P = 0), -Delta
//   tok [B, Np]                  token at the site (-1: none)
// A workgroup of NTH threads takes NTH consecutive sites of one (b, h) (Np is
// a multiple of 256), one site per thread. Every gather (the site's q, dO and
// O_glob rows, its (cos, sin) rows, gate and lse) goes out before any is
// used. The 32-row blocks are written straight from registers; the
// transposed blocks go through one LDS buffer, q~ first and dO_glob after
// it, so that each lane then stores one whole 16-byte chunk (8 sites of one
// channel) and a wave's stores are contiguous.
template <int D>
__global__ __launch_bounds__(D == 48 ? 256 : 128) void k_bwd_prep_mfma(
    Geo g, const void *geom, const bf16 *__restrict__ q, const bf16 *__restrict__ gate,
    const bf16 *__restrict__ dout, const bf16 *__restrict__ oglob, const float *__restrict__ lse,
    bf16 *qn, bf16 *qt, bf16 *dn, bf16 *dt, float *lse_p, float *dl_p, int32_t *tok, int Np) {
  constexpr int DA = D / 3, NCH = D / 8;
  constexpr int NTH = D == 48 ? 256 : 128;
  constexpr int PITCH = D + 8;  // LDS row pitch (elements): 16-byte rows, fewer bank conflicts
  // one staging buffer, used for q~ and then for dO_glob, so that more
  // workgroups fit a CU
  __shared__ __attribute__((aligned(16))) bf16 sQ[NTH * PITCH];
  // Workgroups at D = 48: (batch, site chunk, head) with the heads
  // innermost, so that the workgroups reading the heads of the same tokens
  // run together on one XCD and share the token rows' cache lines in its L2
  // (a head's 96-byte slice shares its 128-byte lines with its neighbours;
  // 119 -> 98 us on the 65,536-token volume). At D = 96 that order measured
  // slower (435 -> 525 us on the anisotropic volume), and (batch, head) stays
  // outermost.
  const int w = D == 48 ? xcd_remap(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int nchunk = Np / NTH;
  int h, b, pbase;
  if constexpr (D == 48) {
    h = w % g.H;
    b = w / (g.H * nchunk);
    pbase = ((w / g.H) % nchunk) * NTH;
  } else {
    h = (w / nchunk) % g.H;
    b = w / (g.H * nchunk);
    pbase = (w % nchunk) * NTH;
  }
  const int p = pbase + (int)threadIdx.x;  // pbase: first site of the workgroup
  const int64_t bh = (int64_t)b * g.H + h;
  const int64_t t = bh * Np + p;  // ((b*H + h) * Np + p)
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int i = p < g.N ? slot_get(g, slot, p) : -1;
  if (h == 0) tok[(int64_t)b * Np + p] = i;
  const int c3[3] = {p / (g.Y * g.X), (p / g.X) % g.Y, p % g.X};
  const int64_t row = ((int64_t)b * g.N + max(i, 0)) * g.H + h;
  const float qscale = g.scale * kLog2e;
  // Every load goes out before any is used, without branches: a site with
  // no token reads token 0's row (its results are replaced by zeros below).
  bf16x8 raw[NCH], draw[NCH], oraw[NCH];
  float2 cs[D / 2];
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    raw[c] = *reinterpret_cast<const bf16x8 *>(q + row * D + 8 * c);
    draw[c] = *reinterpret_cast<const bf16x8 *>(dout + row * D + 8 * c);
    oraw[c] = *reinterpret_cast<const bf16x8 *>(oglob + row * D + 8 * c);
  }
#pragma unroll
  for (int pp = 0; pp < D / 2; pp++) {
    const int a = pp / (DA / 2);  // the axis of channel pair pp
    cs[pp] = rope_cs(tab, g, a, c3[a], pp % (DA / 2));
  }
  const float graw = (float)gate[row], lraw = lse[row];
  const float gg = i >= 0 ? 1.0f / (1.0f + expf(-graw)) : 0.f;
  float dl = 0.f;
  bf16x8 dvs[NCH];  // dO_glob, staged after q~
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    bf16x8 qv, dv;
    if (i >= 0) {
#pragma unroll
      for (int u = 0; u < 4; u++) {
        float x0 = (float)raw[c][2 * u], x1 = (float)raw[c][2 * u + 1];
        rotate(x0, x1, cs[4 * c + u]);
        qv[2 * u] = (bf16)(x0 * qscale);
        qv[2 * u + 1] = (bf16)(x1 * qscale);
      }
#pragma unroll
      for (int e = 0; e < 8; e++) {
        dv[e] = (bf16)(gg * (float)draw[c][e]);
        dl += (float)dv[e] * (float)oraw[c][e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; e++) qv[e] = dv[e] = (bf16)0.0f;
    }
    const int64_t nb = (((bh * (Np / 32) + p / 32) * NCH + c) * 32 + p % 32) * 8;
    *reinterpret_cast<bf16x8 *>(qn + nb) = qv;
    *reinterpret_cast<bf16x8 *>(dn + nb) = dv;
    *reinterpret_cast<bf16x8 *>(&sQ[threadIdx.x * PITCH + 8 * c]) = qv;
    dvs[c] = dv;
  }
  lse_p[t] = i >= 0 ? -lraw : -INFINITY;
  dl_p[t] = -dl;
  // chunk (g8, d) of the workgroup: channel d of its sites 8*g8 .. 8*g8 + 7
  auto transpose_out = [&](bf16 *dst) {
#pragma unroll
    for (int r = 0; r < NCH; r++) {
      const int e = (int)threadIdx.x + NTH * r;
      const int g8 = e / D, d = e % D;
      bf16x8 x;
#pragma unroll
      for (int k = 0; k < 8; k++) x[k] = sQ[(8 * g8 + k) * PITCH + d];
      const int64_t tb = ((bh * (Np / 8) + pbase / 8 + g8) * D + d) * 8;
      *reinterpret_cast<bf16x8 *>(dst + tb) = x;
    }
  };
  __syncthreads();
  transpose_out(qt);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NCH; c++) *reinterpret_cast<bf16x8 *>(&sQ[threadIdx.x * PITCH + 8 * c]) = dvs[c];
  __syncthreads();
  transpose_out(dt);
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
  constexpr int KD = D / 16, NCH = D / 8, NSUB = TS / 32;
  // dq rows: DF whole 32-channel tiles, and with T16 a last tile of 16
  // channels, done as two 16x16x32 products (one per 16 queries) so that no
  // matrix-core cycle goes to padding channels
  constexpr int DF = D / 32;
  constexpr bool T16 = D % 32 == 16;
  static_assert(D % 32 == 0 || T16, "channels in whole 16-channel tiles");
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
  // -lse and -Delta of the lane's query, in every register: the start value
  // of its score and dP columns
  f32x16 lq[G], dq[G];
  f32x16 acc[G][DF];
  f32x4 accT[2] = {};  // the 16-channel tile (T16): queries 16*half ..
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
    const float nl = lse_p[(int64_t)bh * Np + p[gi]], nd = dl_p[(int64_t)bh * Np + p[gi]];
#pragma unroll
    for (int j = 0; j < 16; j++) {
      lq[gi][j] = nl;
      dq[gi][j] = nd;
    }
#pragma unroll
    for (int t = 0; t < DF; t++)
#pragma unroll
      for (int j = 0; j < 16; j++) acc[gi][t][j] = 0.f;
  }

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
        s[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[gi][c], c == 0 ? lq[gi] : s[gi], 0, 0, 0);
        dp[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[gi][c], c == 0 ? dq[gi] : dp[gi], 0, 0, 0);
      }
    }
#pragma unroll
    for (int gi = 0; gi < G; gi++) {
      // register j <-> summary mbase + 16*(j/8) + 8*hi + j%8
      bf16x8 tf[2];
#pragma unroll
      for (int j = 0; j < 16; j++) {
        float t = __builtin_amdgcn_exp2f(s[gi][j]) * dp[gi][j];
        if constexpr (decltype(mask)::value)
          t = (mbase + 16 * (j >> 3) + 8 * hi + (j & 7) < g.M) ? t : 0.f;
        tf[j >> 3][j & 7] = (bf16)t;
      }
#pragma unroll
      for (int t = 0; t < DF; t++) {
        const int d = 32 * t + l32;
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++) {
          const bf16x8 kf2 = T[(4 * sub + 2 * c2 + hi) * D + d];
          acc[gi][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf2, tf[c2], acc[gi][t], 0, 0, 0);
        }
      }
    }
  };
  if constexpr (G == 1 && NSUB == 4) {
    // Three-stage software pipeline over 32-summary sub-tiles, as in the
    // forward: step j issues the dq products of sub-tile j, runs the vector
    // work of sub-tile j+1 (dT = exp2(t - lse) (dP - Delta), rounded to bf16)
    // and issues the score and dP products of sub-tile j+2, so the matrix
    // products of a step depend on none of its vector instructions. The
    // operands of the next step's products are read from LDS right after
    // this step's products take the current ones.
    //
    // Tile u (buffer u & 1) holds the k_sum and v_sum rows of sub-tiles
    // 4u .. 4u+3 and the channel-major k_sum of sub-tiles 4u-2 .. 4u+1, two
    // behind: step j reads the rows of sub-tile j+3 and the channel-major
    // part of sub-tile j+1, both at position (j+3) % 4 of tile (j+3) / 4.
    // So both switch tiles at the steps with (j+3) % 4 == 0, after one
    // barrier, which also ends every read of the tile before; the loads of
    // the tile after go into that tile's buffers right after it, four steps
    // ahead of their use. Summaries at or past M get dT = 0 (a select, so
    // whatever a clamped or stale LDS row held is discarded), and the steps
    // past the last sub-tile issue no dq products.
    // An iteration is two tiles (2 * NSUB steps), so that every buffer
    // choice is known at compile time: the compiler can then tell the LDS
    // reads from the loads into the other buffer and does not wait for those.
    const int S = M32;                                  // sub-tiles with summaries
    const int NIT = (S + 2 * NSUB - 1) / (2 * NSUB);    // iterations
    const int NTL = (S + 2 + NSUB - 1) / NSUB;          // tiles to load
    const int MF = g.M / 32;                            // sub-tiles wholly below M
    const int IT_CLEAN = MF >= 1 ? min(NIT, (MF - 1) / (2 * NSUB)) : 0;
    auto issue_p = [&](int tt, bf16x8 *dK, bf16x8 *dV, bf16x8 *dT) {
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
          const int g8 = min(max(tt * NJ8 - 8 + rt_j8[r], 0), 4 * M32 - 1);  // two sub-tiles back
          const uint32_t o = (uint32_t)(g8 * D + rt_d[r]) * 16;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rkt, (lds_ptr)&dT[NTH * r + 64 * wv], 16, o, 0, 0, 0);
        }
      }
    };
    f32x16 s2[2], dp2[2];  // scores and dP, by parity of the sub-tile
    bf16x8 tf2[2][2];      // dT, by parity of the sub-tile
    bf16x8 kf[KD], vf[KD]; // score / dP operands of the next products
    bf16x8 tq[DF][2];      // dq operands of the next products
    bf16x8 tqt;            // ... of the 16-channel tile (T16)
    auto read_kv = [&](const bf16x8 *K, const bf16x8 *V, int pos) {
#pragma unroll
      for (int c = 0; c < KD; c++) {
        kf[c] = K[(2 * c + hi) * TS + 32 * pos + l32];
        vf[c] = V[(2 * c + hi) * TS + 32 * pos + l32];
      }
    };
    auto read_t = [&](const bf16x8 *T, int ls) {
#pragma unroll
      for (int t = 0; t < DF; t++) {
        const int d = 32 * t + l32;
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++) tq[t][c2] = T[(4 * ls + 2 * c2 + hi) * D + d];
      }
      if constexpr (T16) {
        // lane: channel 32*DF + lane%16, k block lane/16 <-> summaries
        // 8*sigma(lane/16) .. +7 of the sub-tile (sigma swaps the two bits;
        // the order the lane swap in qprod leaves dT in)
        const int kb = lane >> 4;
        tqt = T[(4 * ls + ((kb >> 1) | ((kb & 1) << 1))) * D + 32 * DF + (lane & 15)];
      }
    };
    auto sd = [&](f32x16 &sx, f32x16 &dx) {
#pragma unroll
      for (int c = 0; c < KD; c++) {
        sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[0][c], c == 0 ? lq[0] : sx, 0, 0, 0);
        dx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c], df[0][c], c == 0 ? dq[0] : dx, 0, 0, 0);
      }
    };
    // register e <-> summary mbase + 16*(e/8) + 8*hi + e%8
    // (built a pair at a time, so each pair is one packed conversion)
    auto tvec = [&](const f32x16 &sx, const f32x16 &dx, bf16x8 *tx, int mbase, auto mask) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float t0 = __builtin_amdgcn_exp2f(sx[e]) * dx[e];
        float t1 = __builtin_amdgcn_exp2f(sx[e + 1]) * dx[e + 1];
        if constexpr (decltype(mask)::value) {
          const int m0 = mbase + 16 * (e >> 3) + 8 * hi + (e & 7);
          t0 = m0 < g.M ? t0 : 0.f;
          t1 = m0 + 1 < g.M ? t1 : 0.f;
        }
        bf16x2 pr;
        pr[0] = (bf16)t0;
        pr[1] = (bf16)t1;
        tx[e >> 3] = set_pair(tx[e >> 3], (e & 7) / 2, pr);
      }
    };
    auto qprod = [&](bf16x8 *tx) {
#pragma unroll
      for (int t = 0; t < DF; t++)
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++)
          acc[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[t][c2], tx[c2], acc[0][t], 0, 0, 0);
      if constexpr (T16) {
        // Lane (n, hi) holds query n, summaries 16*c2 + 8*hi .. +7 in
        // operand c2; v_permlane16_swap of (c2 = 0, c2 = 1) leaves queries
        // 0..15 in the first and 16..31 in the second, in lane row r the
        // summaries 8*sigma(r) .. +7: the B operand of a 16x16x32 product.
        // In place: the products above have taken the first layout, and
        // dT of this sub-tile has no later reader.
        swap_rows16(tx);
#pragma unroll
        for (int hf = 0; hf < 2; hf++)
          accT[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tqt, tx[hf], accT[hf], 0, 0, 0);
      }
    };
    issue_p(0, sK0, sV0, sT0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (NTL > 1) issue_p(1, sK1, sV1, sT1);
    read_kv(sK0, sV0, 0);
    sd(s2[0], dp2[0]);
    read_kv(sK0, sV0, 1);
    sd(s2[1], dp2[1]);
    tvec(s2[0], dp2[0], tf2[0], 0, std::true_type{});
    read_kv(sK0, sV0, 2);
    read_t(sT0, 2);  // sub-tile 0 sits at position 2 of tile 0's channel-major part
    auto step = [&](int it, auto jc, auto mc) {
      constexpr int JJ = decltype(jc)::value;  // step within the iteration
      constexpr int POS = (JJ + 3) % NSUB, P = JJ & 1;
      constexpr int KB = ((JJ + 3) / NSUB) & 1;  // buffer of tile (j+3) / NSUB
      const int KT = 2 * it + (JJ + 3) / NSUB;
      const int j = 2 * NSUB * it + JJ;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (POS == 0) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads landed, its LDS reads done
        __syncthreads();
        if (KT + 1 < NTL) issue_p(KT + 1, KB ? sK0 : sK1, KB ? sV0 : sV1, KB ? sT0 : sT1);
      }
      const bf16x8 *K = KB ? sK1 : sK0, *V = KB ? sV1 : sV0, *T = KB ? sT1 : sT0;
      // sub-tile j; past the last sub-tile its operands may come from a
      // buffer never loaded (0 * NaN would reach the sums), so skip it
      if constexpr (!decltype(mc)::value) qprod(tf2[P]);
      else if (j < S) qprod(tf2[P]);
      sd(s2[P], dp2[P]);      // sub-tile j+2
      read_kv(K, V, POS);     // sub-tile j+3
      tvec(s2[P ^ 1], dp2[P ^ 1], tf2[P ^ 1], 32 * (j + 1), mc);  // sub-tile j+1
      read_t(T, POS);         // sub-tile j+1
      __builtin_amdgcn_sched_barrier(0);
    };
    auto iteration = [&](int it, auto mc) {
      step(it, std::integral_constant<int, 0>{}, mc);
      step(it, std::integral_constant<int, 1>{}, mc);
      step(it, std::integral_constant<int, 2>{}, mc);
      step(it, std::integral_constant<int, 3>{}, mc);
      step(it, std::integral_constant<int, 4>{}, mc);
      step(it, std::integral_constant<int, 5>{}, mc);
      step(it, std::integral_constant<int, 6>{}, mc);
      step(it, std::integral_constant<int, 7>{}, mc);
    };
    int it = 0;
    for (; it < IT_CLEAN; it++) iteration(it, std::false_type{});
    for (; it < NIT; it++) iteration(it, std::true_type{});
    __builtin_amdgcn_s_waitcnt(0);
  } else {
  static_assert(!T16, "the one-tile-at-a-time form has whole 32-channel tiles only");
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
          s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[0][c], c == 0 ? lq[0] : s[sub], 0, 0, 0);
          dp[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[0][c], c == 0 ? dq[0] : dp[sub], 0, 0, 0);
        }
#pragma unroll
      for (int sub = 0; sub < NSUB; sub++) {
        bf16x8 tf[2];
#pragma unroll
        for (int j = 0; j < 16; j++)
          tf[j >> 3][j & 7] = (bf16)(__builtin_amdgcn_exp2f(s[sub][j]) * dp[sub][j]);
#pragma unroll
        for (int t = 0; t < DF; t++) {
          const int d = 32 * t + l32;
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
  }
  // lane: query site p (column l32), rows d = 32t + 8jj + 4hi + u
#pragma unroll
  for (int gi = 0; gi < G; gi++) {
    const int i = p[gi] < g.N ? tok[(int64_t)b * Np + p[gi]] : -1;
    if (i < 0) continue;
    float *orow = dqg + (((int64_t)b * g.N + i) * g.H + h) * D;
#pragma unroll
    for (int t = 0; t < DF; t++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int d = 32 * t + 8 * jj + 4 * hi;
        f32x4 o4;
#pragma unroll
        for (int u = 0; u < 4; u++) o4[u] = g.scale * acc[gi][t][4 * jj + u];
        *reinterpret_cast<f32x4 *>(orow + d) = o4;
      }
  }
  if constexpr (T16) {
    // 16x16 blocks: lane: query site 16*half + lane%16 of the wave's 32,
    // channels 32*DF + 4*(lane/16) .. +3
    static_assert(G == 1, "one query group per wave");
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      const int pt = tile * (NW * 32) + wv * 32 + 16 * hf + (lane & 15);
      const int i = pt < g.N ? tok[(int64_t)b * Np + pt] : -1;
      if (i < 0) continue;
      f32x4 o4;
#pragma unroll
      for (int u = 0; u < 4; u++) o4[u] = g.scale * accT[hf][u];
      *reinterpret_cast<f32x4 *>(dqg + (((int64_t)b * g.N + i) * g.H + h) * D + 32 * DF +
                                 4 * (lane >> 4)) = o4;
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
  constexpr int KD = D / 16, NCH = D / 8, NSUB = TQ / 32, NJ8 = TQ / 8;
  // dK / dV columns: DF whole 32-channel tiles, and with T16 a last tile of
  // 16 channels, done as two 16x16x32 products (one per 16 summaries) so
  // that no matrix-core cycle goes to padding channels
  constexpr int DF = D / 32;
  constexpr bool T16 = D % 32 == 16;
  static_assert(D % 32 == 0 || T16, "channels in whole 16-channel tiles");
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
  f32x16 aK[DF], aV[DF];
  f32x4 aKt[2], aVt[2];  // the 16-channel tile: summaries 16*half ..
#pragma unroll
  for (int t = 0; t < DF; t++)
#pragma unroll
    for (int j = 0; j < 16; j++) aK[t][j] = aV[t][j] = 0.f;
#pragma unroll
  for (int hf = 0; hf < 2; hf++)
#pragma unroll
    for (int j = 0; j < 4; j++) aKt[hf][j] = aVt[hf][j] = 0.f;

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
  // buffer resources of head h's slices: both query layouts are Np * D
  // elements per head
  auto rsrc = [&](const bf16 *base, int h) {
    return buffer_rsrc(base + ((int64_t)b * g.H + h) * Np * D, Np * D * 2);
  };
  // the row-layout part of iteration it's query tile (q~, dO, -lse, -Delta)
  auto issue_a = [&](int it, bf16x8 *dQ, bf16x8 *dD, float *dL, float *dDl) {
    const int h = hk * g.G + it / nq, qtile = qt0 + it % nq;
    const __amdgpu_buffer_rsrc_t rq = rsrc(qn, h), rd = rsrc(dn, h);
#pragma unroll
    for (int r = 0; r < RN; r++) {
      if (NTH * r + 64 * wv < NNC) {
        const uint32_t o = (uint32_t)((qtile * NSUB + rn_sub[r]) * (NCH * 256) + rn_in[r]) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_ptr)&dQ[NTH * r + 64 * wv], 16, o, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_ptr)&dD[NTH * r + 64 * wv], 16, o, 0, 0, 0);
      }
    }
    // per-site statistics: wave 0 -lse, wave 1 -Delta (4 bytes a lane)
    if (wv < 2) {
      const int64_t bh = (int64_t)b * g.H + h;
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc((wv == 0 ? lse_p : dl_p) + bh * Np, Np * 4);
      const uint32_t o = (uint32_t)(qtile * TQ + min(lane, TQ - 1)) * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(wv == 0 ? dL : dDl), 4, o, 0, 0, 0);
    }
  };
  // the channel-major part (q~ and dO, 8 sites per chunk)
  auto issue_b = [&](int it, bf16x8 *dQT, bf16x8 *dDT) {
    const int h = hk * g.G + it / nq, qtile = qt0 + it % nq;
    const __amdgpu_buffer_rsrc_t rqt = rsrc(qt, h), rdt = rsrc(dt, h);
#pragma unroll
    for (int r = 0; r < RTT; r++) {
      if (NTH * r + 64 * wv < NTC) {
        const uint32_t o = (uint32_t)((qtile * NJ8 + rt_j8[r]) * D + rt_d[r]) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rqt, (lds_ptr)&dQT[NTH * r + 64 * wv], 16, o, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rdt, (lds_ptr)&dDT[NTH * r + 64 * wv], 16, o, 0, 0, 0);
      }
    }
  };
  auto issue = [&](int it, bf16x8 *dQ, bf16x8 *dD, bf16x8 *dQT, bf16x8 *dDT, float *dL,
                   float *dDl) {
    issue_a(it, dQ, dD, dL, dDl);
    issue_b(it, dQT, dDT);
  };
  if constexpr (NSUB == 2) {
    // Three-stage pipeline over the 32-query sub-tiles of all iterations.
    // Step j issues the dK/dV products of sub-tile j-2, runs the softmax of
    // sub-tile j-1 while they execute, then issues the score and dP products
    // of sub-tile j, and reads from LDS the fragments of the next step's
    // products: the row layout of sub-tile j+1 and the channel-major layout
    // of sub-tile j-1. Those two are two sub-tiles apart, so the
    // channel-major tiles trail the row tiles by one: tile u holds the row
    // part of iteration u and the channel-major part of iteration u-1, in
    // buffer u & 1. Odd steps switch to tile u = (j+1)/2 after their score
    // products (which read tile u-1): a barrier publishes tile u, and the
    // loads of tile u+1 then go into the buffers of tile u-1. Only one score
    // tile is live at a time: the softmax empties it before the start values
    // of the next sub-tile go in.
    const int S = 2 * ntile;
    auto issue_tile = [&](int u, auto par) {
      constexpr int P = decltype(par)::value;
      if (u < ntile) issue_a(u, P ? sQ1 : sQ0, P ? sD1 : sD0, P ? sL1 : sL0, P ? sDl1 : sDl0);
      if (u >= 1 && u - 1 < ntile) issue_b(u - 1, P ? sQT1 : sQT0, P ? sDT1 : sDT0);
    };
    f32x16 s, dp;                // scores and dP of one sub-tile
    bf16x8 pa[2], ta[2];         // P and dT of the sub-tile the softmax last produced
    bf16x8 qa[KD], da[KD];       // score / dP operands of the next sub-tile
    bf16x8 qb[DF][2], db[DF][2]; // dK / dV operands of the next sub-tile
    bf16x8 qbt, dbt;             // ... of its 16-channel tile (T16)
    // the q~ and dO fragments of the sub-tile at position POS of a tile
    auto read_sd = [&](auto par, auto pos) {
      constexpr int P = decltype(par)::value, POS = decltype(pos)::value;
      const bf16x8 *Q = P ? sQ1 : sQ0, *Dd = P ? sD1 : sD0;
#pragma unroll
      for (int c = 0; c < KD; c++) {
        qa[c] = Q[(2 * c + hi) * TQ + 32 * POS + l32];
        da[c] = Dd[(2 * c + hi) * TQ + 32 * POS + l32];
      }
    };
    // -lse and -Delta of its sites, the start values of the products:
    // register 8*c2 + e of half hi <-> site 32*POS + 16*c2 + 8*hi + e
    auto read_init = [&](auto par, auto pos) {
      constexpr int P = decltype(par)::value, POS = decltype(pos)::value;
      const float *L = P ? sL1 : sL0, *Dl = P ? sDl1 : sDl0;
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++)
#pragma unroll
        for (int hq = 0; hq < 2; hq++) {
          const int q0 = 32 * POS + 16 * c2 + 8 * hi + 4 * hq;
          const f32x4 l4 = *reinterpret_cast<const f32x4 *>(L + q0);
          const f32x4 d4 = *reinterpret_cast<const f32x4 *>(Dl + q0);
#pragma unroll
          for (int u = 0; u < 4; u++) {
            s[8 * c2 + 4 * hq + u] = l4[u];
            dp[8 * c2 + 4 * hq + u] = d4[u];
          }
        }
    };
    auto read_kv = [&](auto par, auto pos) {
      constexpr int P = decltype(par)::value, POS = decltype(pos)::value;
      const bf16x8 *QT = P ? sQT1 : sQT0, *DTt = P ? sDT1 : sDT0;
#pragma unroll
      for (int t = 0; t < DF; t++) {
        const int d = 32 * t + l32;
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++) {
          const int j8 = 4 * POS + 2 * c2 + hi;
          qb[t][c2] = QT[j8 * D + d];
          db[t][c2] = DTt[j8 * D + d];
        }
      }
      if constexpr (T16) {
        // lane: channel 32*DF + lane%16, k block lane/16 <-> sites
        // 8*sigma(lane/16) .. +7 of the sub-tile (sigma swaps the two bits;
        // the order the lane swap below leaves P and dT in)
        const int kb = lane >> 4;
        const int j8 = 4 * POS + ((kb >> 1) | ((kb & 1) << 1));
        qbt = QT[j8 * D + 32 * DF + (lane & 15)];
        dbt = DTt[j8 * D + 32 * DF + (lane & 15)];
      }
    };
    issue_tile(0, std::integral_constant<int, 0>{});
    issue_tile(1, std::integral_constant<int, 1>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (S > 0) read_sd(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    // one step; JJ = position in a group of four steps (two tiles)
    auto step = [&](int grp, auto jc, auto fc) {
      constexpr int JJ = decltype(jc)::value;
      constexpr bool FULL = decltype(fc)::value;  // every part of the step exists
      constexpr int TC = (JJ / 2) & 1, PC = JJ % 2;              // tile, position of sub-tile j
      constexpr int TN = ((JJ + 1) / 2) & 1, PN = (JJ + 1) % 2;  // of sub-tile j+1
      constexpr bool SWITCH = PN == 0;
      const int j = 4 * grp + JJ;
      __builtin_amdgcn_sched_barrier(0);
      if (FULL || (j >= 2 && j - 2 < S)) {
#pragma unroll
        for (int t = 0; t < DF; t++)
#pragma unroll
          for (int c2 = 0; c2 < 2; c2++) {
            aK[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[c2], qb[t][c2], aK[t], 0, 0, 0);
            aV[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[c2], db[t][c2], aV[t], 0, 0, 0);
          }
        if constexpr (T16) {
          // Lane (n, hi) holds summary n, sites 16*c2 + 8*hi .. +7 in
          // operand c2. v_permlane16_swap trades lanes 16..31 / 48..63 of
          // its first operand with lanes 0..15 / 32..47 of its second, so
          // with (c2 = 0, c2 = 1) as operands the first result holds
          // summaries 0..15 and the second summaries 16..31, in every lane
          // row r = lane/16 the sites 8*sigma(r) .. +7: the A operand of a
          // 16x16x32 product. The swap goes in place, after the products
          // above have taken the first layout.
          swap_rows16(pa);
          swap_rows16(ta);
#pragma unroll
          for (int hf = 0; hf < 2; hf++) {
            aKt[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta[hf], qbt, aKt[hf], 0, 0, 0);
            aVt[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[hf], dbt, aVt[hf], 0, 0, 0);
          }
        }
      }
      if (FULL || (j >= 1 && j - 1 < S)) {
        // built a pair at a time, so each pair is one packed conversion
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(s[8 * c2 + e]);
            const float p1 = __builtin_amdgcn_exp2f(s[8 * c2 + e + 1]);
            bf16x2 pp, tp;
            pp[0] = (bf16)p0;
            pp[1] = (bf16)p1;
            tp[0] = (bf16)(p0 * dp[8 * c2 + e]);
            tp[1] = (bf16)(p1 * dp[8 * c2 + e + 1]);
            pa[c2] = set_pair(pa[c2], e / 2, pp);
            ta[c2] = set_pair(ta[c2], e / 2, tp);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
      // The next step's dK / dV operands (sub-tile j-1) are read as early as
      // their tile allows: in a step without a switch that tile is published
      // already, so they go out before this step's score products.
      if constexpr (!SWITCH)
        if (FULL || (j >= 1 && j - 1 < S))
          read_kv(std::integral_constant<int, TN>{}, std::integral_constant<int, PN>{});
      if (FULL || j < S)
        read_init(std::integral_constant<int, TC>{}, std::integral_constant<int, PC>{});
      if constexpr (SWITCH) {
        // read_init above was the last read of tile u-1; the score products
        // below use operands already in registers
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads landed, its LDS reads done
        __syncthreads();
        issue_tile(2 * grp + (JJ + 1) / 2 + 1,
                   std::integral_constant<int, ((JJ + 1) / 2 + 1) & 1>{});
        if (FULL || (j >= 1 && j - 1 < S))
          read_kv(std::integral_constant<int, TN>{}, std::integral_constant<int, PN>{});
      }
      if (FULL || j < S) {
#pragma unroll
        for (int c = 0; c < KD; c++) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[c], kb[c], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[c], vb[c], dp, 0, 0, 0);
        }
      }
      if (FULL || j + 1 < S)
        read_sd(std::integral_constant<int, TN>{}, std::integral_constant<int, PN>{});
      __builtin_amdgcn_sched_barrier(0);
    };
    // groups whose four steps are whole (2 <= j and j + 1 < S) run without
    // checks; the first and the last ones check each part
    auto group = [&](int grp, auto fc) {
      step(grp, std::integral_constant<int, 0>{}, fc);
      step(grp, std::integral_constant<int, 1>{}, fc);
      step(grp, std::integral_constant<int, 2>{}, fc);
      step(grp, std::integral_constant<int, 3>{}, fc);
    };
    const int ngrp = (S + 2 + 3) / 4;  // steps 0 .. S+1
    int grp = 0;
    if (ngrp > 0) group(grp++, std::false_type{});
    for (; 4 * grp + 4 < S; grp++) group(grp, std::true_type{});
    for (; grp < ngrp; grp++) group(grp, std::false_type{});
  } else {
    static_assert(!T16, "the one-tile-at-a-time form has whole 32-channel tiles only");
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
      // C[query rows][summary columns]: row r holds query site swap23(r), so
      // register 8*c2 + e of half hi <-> site 32*sub + 16*c2 + 8*hi + e. The
      // products start from -lse and -Delta of those sites.
      f32x16 s[NSUB], dp[NSUB];
  #pragma unroll
      for (int sub = 0; sub < NSUB; sub++) {
  #pragma unroll
        for (int c2 = 0; c2 < 2; c2++)
  #pragma unroll
          for (int hq = 0; hq < 2; hq++) {
            const int q0 = 32 * sub + 16 * c2 + 8 * hi + 4 * hq;
            const f32x4 l4 = *reinterpret_cast<const f32x4 *>(L + q0);
            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(Dl + q0);
  #pragma unroll
            for (int u = 0; u < 4; u++) {
              s[sub][8 * c2 + 4 * hq + u] = l4[u];
              dp[sub][8 * c2 + 4 * hq + u] = d4[u];
            }
          }
  #pragma unroll
        for (int c = 0; c < KD; c++) {
          const bf16x8 qa = Q[(2 * c + hi) * TQ + 32 * sub + l32];
          const bf16x8 da = Dd[(2 * c + hi) * TQ + 32 * sub + l32];
          s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb[c], s[sub], 0, 0, 0);
          dp[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vb[c], dp[sub], 0, 0, 0);
        }
      }
  #pragma unroll
      for (int sub = 0; sub < NSUB; sub++) {
        bf16x8 pa[2], ta[2];
  #pragma unroll
        for (int c2 = 0; c2 < 2; c2++)
  #pragma unroll
          for (int e = 0; e < 8; e++) {
            const float pr = __builtin_amdgcn_exp2f(s[sub][8 * c2 + e]);
            pa[c2][e] = (bf16)pr;
            ta[c2][e] = (bf16)(pr * dp[sub][8 * c2 + e]);
          }
  #pragma unroll
        for (int t = 0; t < DF; t++) {
          const int d = 32 * t + l32;
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
  }
  if (!wave_live) return;
  // lane: channel column 32t + l32, rows = summaries 8jj + 4hi + u of the group
  const int64_t base = (((int64_t)split * g.B * g.Hkv + bk) * g.M) * D;
#pragma unroll
  for (int t = 0; t < DF; t++) {
    const int d = 32 * t + l32;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int m = m32 * 32 + (j >> 2) * 8 + hi * 4 + (j & 3);
      if (m < g.M) {
        dks_part[base + (int64_t)m * D + d] = kLn2 * aK[t][j];  // s / (s log2 e)
        dvs_part[base + (int64_t)m * D + d] = aV[t][j];
      }
    }
  }
  if constexpr (T16) {
    // 16x16 blocks: lane: channel 32*DF + lane%16, summaries 16*half +
    // 4*(lane/16) + u
    const int d = 32 * DF + (lane & 15);
#pragma unroll
    for (int hf = 0; hf < 2; hf++)
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int m = m32 * 32 + 16 * hf + 4 * (lane >> 4) + u;
        if (m < g.M) {
          dks_part[base + (int64_t)m * D + d] = kLn2 * aKt[hf][u];
          dvs_part[base + (int64_t)m * D + d] = aVt[hf][u];
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
    constexpr int NTH = D == 48 ? 256 : 128;  // divides Np
    const int64_t n = (int64_t)g.B * g.H * Np;
    hipLaunchKernelGGL((k_bwd_prep_mfma<D>), dim3((unsigned)(n / NTH)), dim3(NTH), 0, s, g,
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
  if (g.D == 48) return run_bwd_global_mfma<48, 128, 64, 4, 1, 4>(g, a, m, s);
  return run_bwd_global_mfma<96, 64, 32, 4, 1, 4>(g, a, m, s);
}

}  // namespace pk
