// Query-to-summary attention on bf16 matrix cores (Geometry Matters in Packed
// 3D Attention, project page Ch. 3, Contract 2; paper summary §3.5, §B.10).
//
// The global branch is a dense contraction -- every query against all M
// summaries -- so it runs as a flash-style loop on v_mfma_f32_32x32x16_bf16
// with an fp32 online softmax and never forms the token x summary score
// matrix (paper summary §3.5).
//
// Layout of the work. A workgroup of 4 waves owns 128 consecutive tokens
// (packed order) of one (batch, head); a wave owns 32 of them. Summary tiles
// of 64 rows of k_sum and v_sum go through LDS (v_sum stored transposed).
// Per 32-summary sub-tile a wave computes the TRANSPOSED scores
// S^T = Ksum * Q~^T (32 summaries x 32 queries), so every lane holds 16
// scores of ONE query and the running maximum, the rescale and the final
// normalisation are lane-local. The k_sum rows are loaded in the order
// r -> r with bits 2 and 3 swapped, which makes the score registers come out
// exactly in the operand order of the next product O^T += Vsum^T * P^T: the
// probabilities go from registers straight into the matrix core, no shuffle.
//
// Softmax details. Scores are in log2 units (the query is pre-multiplied by
// scale*log2(e)). Subtracting a running maximum only guards exp against
// overflow and underflow; fp32 and bf16 share one 8-bit exponent range, so
// as long as every score stays below 2^7 and the denominator stays well
// above the underflow limit, p = exp2(s) with no maximum at all gives the
// same softmax up to rounding. That is the fast path: no maximum, no
// rescale, the matrix core accumulates straight from exp2. For D = 48 the
// output tile has 16 spare rows; row 48 of the transposed value tile is all
// ones, so the matrix core also returns the denominator. A query whose
// denominator comes out non-finite or below 2^-100 is recomputed by an exact
// two-pass path (maximum first, then the sums with the maximum subtracted)
// that reads the summaries straight from global memory; queries that passed
// keep their fast-path result. The choice is made per query, and each
// query's arithmetic depends only on its own row and the summaries, never on
// which tokens share its tile, so a repack of the tokens permutes the output
// bit for bit.
#include "launch.hpp"

namespace pk {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTS = 64;       // summaries per LDS tile
constexpr int kWaves = 4;

__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
}  // namespace

// G = 32-query groups per wave; both groups share every LDS fragment read.
template <int D, int G>
__global__ __launch_bounds__(256, D == 48 ? 2 : 3) void k_global_mfma(Geo g, const void *geom,
                                                        const int32_t *__restrict__ coords,
                                                        const bf16 *__restrict__ q,
                                                        const bf16 *__restrict__ ks,
                                                        const bf16 *__restrict__ vs,
                                                        bf16 *__restrict__ out, int ntiles) {
  constexpr int DA = D / 3;
  constexpr int KD = D / 16;                // 16-deep steps of Ksum * Q~^T
  constexpr bool ONES = (D % 32) != 0;      // spare output rows carry the denominator
  constexpr int DT = (D + 31) / 32;         // 32-row tiles of O^T
  constexpr int DPAD = DT * 32;
  constexpr int KP = D + 8;                 // LDS pitch of a Ksum row (elements)
  constexpr int VP = kTS + 8;               // LDS pitch of a Vsum^T row (elements)
  constexpr int QPW = 32 * G;               // queries per wave
  constexpr int NKC = kTS * D / 8;          // 16-byte Ksum chunks per tile
  constexpr int NVC = (kTS / 2) * (D / 8);  // Vsum chunk pairs (two summaries) per tile
  constexpr int KPT = (NKC + 255) / 256;
  constexpr int VPT = (NVC + 255) / 256;
  static_assert(D % 16 == 0 && DA % 8 == 0, "D must be a multiple of 48");
  __shared__ __attribute__((aligned(16))) bf16 sK[2][kTS * KP];
  __shared__ __attribute__((aligned(16))) bf16 sVt[2][DPAD * VP];

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = w % ntiles;
  const int bh = w / ntiles;
  const int h = bh % g.H, b = bh / g.H;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int hi = lane >> 5;  // which half of the wave
  const int64_t sbase = ((int64_t)b * g.H + h) * g.M * D;
  const int tid = threadIdx.x;

  // constant spare rows of the transposed value tiles (never overwritten)
  if constexpr (DPAD > D) {
    for (int e = tid; e < 2 * (DPAD - D) * kTS; e += 256) {
      const int bufi = e / ((DPAD - D) * kTS), rem = e % ((DPAD - D) * kTS);
      const int r = D + rem / kTS, c = rem % kTS;
      sVt[bufi][r * VP + c] = (bf16)((ONES && r == D) ? 1.0f : 0.0f);
    }
  }

  // Query fragments: lane holds channels 16c + 8*hi .. +7 of its query,
  // rotated at the token's own coordinate, scaled, rounded to bf16. A token
  // whose coordinate is off the grid takes no part (zero query, zero output
  // row; only reachable without PACK3D_VALIDATE).
  bf16x8 qf[G][KD];
  bool active[G], cok[G];
  int qi[G];
  {
    const float2 *tab = rope_table(geom, g);
    const float qscale = g.scale * kLog2e;
#pragma unroll
    for (int gi = 0; gi < G; gi++) {
      qi[gi] = tile * (kWaves * QPW) + wv * QPW + gi * 32 + (lane & 31);
      active[gi] = qi[gi] < g.N;
      cok[gi] = false;
      int c3[3] = {0, 0, 0};
      if (active[gi]) {
        c3[0] = coords[3 * (int64_t)qi[gi]];
        c3[1] = coords[3 * (int64_t)qi[gi] + 1];
        c3[2] = coords[3 * (int64_t)qi[gi] + 2];
        cok[gi] = c3[0] >= 0 && c3[1] >= 0 && c3[2] >= 0 && c3[0] < g.Z && c3[1] < g.Y &&
                  c3[2] < g.X;
        if (!cok[gi]) c3[0] = c3[1] = c3[2] = 0;
      }
      const int64_t off = (((int64_t)b * g.N + qi[gi]) * g.H + h) * D;
#pragma unroll
      for (int c = 0; c < KD; c++) {
        const int d0 = 16 * c + 8 * hi;
        const int a = d0 / DA, p0 = (d0 % DA) / 2;
        float x[8];
        if (cok[gi]) {
          const bf16x8 raw = *reinterpret_cast<const bf16x8 *>(q + off + d0);
#pragma unroll
          for (int e = 0; e < 8; e++) x[e] = (float)raw[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; e++) x[e] = 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
          rotate(x[2 * u], x[2 * u + 1], rope_cs(tab, g, a, c3[a], p0 + u));
          qf[gi][c][2 * u] = (bf16)(x[2 * u] * qscale);
          qf[gi][c][2 * u + 1] = (bf16)(x[2 * u + 1] * qscale);
        }
      }
    }
  }

  // Tile staging through registers: global loads for tile t+1 are issued
  // before the arithmetic on tile t and written to the other LDS buffer
  // after it, so one barrier per tile suffices.
  bf16x8 pk[KPT], pv[VPT][2];
  auto load_tile = [&](int m0) {
    const int nm = min(kTS, g.M - m0);
#pragma unroll
    for (int u = 0; u < KPT; u++) {
      const int e = tid + 256 * u;
      const int r = e / (D / 8), ch = e % (D / 8);
      if (e < NKC && r < nm)
        pk[u] = *reinterpret_cast<const bf16x8 *>(ks + sbase + (int64_t)(m0 + r) * D + 8 * ch);
      else
#pragma unroll
        for (int x = 0; x < 8; x++) pk[u][x] = (bf16)0.0f;
    }
#pragma unroll
    for (int u = 0; u < VPT; u++) {
      const int e = tid + 256 * u;
      const int rp = e / (D / 8), ch = e % (D / 8);
#pragma unroll
      for (int y = 0; y < 2; y++) {
        if (e < NVC && 2 * rp + y < nm)
          pv[u][y] = *reinterpret_cast<const bf16x8 *>(vs + sbase + (int64_t)(m0 + 2 * rp + y) * D +
                                                       8 * ch);
        else
#pragma unroll
          for (int x = 0; x < 8; x++) pv[u][y][x] = (bf16)0.0f;
      }
    }
  };
  auto store_tile = [&](int bufi) {
#pragma unroll
    for (int u = 0; u < KPT; u++) {
      const int e = tid + 256 * u;
      if (e < NKC) {
        const int r = e / (D / 8), ch = e % (D / 8);
        *reinterpret_cast<bf16x8 *>(&sK[bufi][r * KP + 8 * ch]) = pk[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; u++) {
      const int e = tid + 256 * u;
      if (e < NVC) {
        const int rp = e / (D / 8), ch = e % (D / 8);
#pragma unroll
        for (int x = 0; x < 8; x++) {
          bf16x2 two;
          two[0] = pv[u][0][x];
          two[1] = pv[u][1][x];
          *reinterpret_cast<bf16x2 *>(&sVt[bufi][(8 * ch + x) * VP + 2 * rp]) = two;
        }
      }
    }
  };

  f32x16 acc[G][DT];
  float lsum[G];
#pragma unroll
  for (int gi = 0; gi < G; gi++) {
#pragma unroll
    for (int t = 0; t < DT; t++)
#pragma unroll
      for (int j = 0; j < 16; j++) acc[gi][t][j] = 0.f;
    lsum[gi] = 0.f;
  }
  const f32x16 zero16 = {};
  const int rowK = swap23(lane & 31);
  const int ntile_s = (g.M + kTS - 1) / kTS;

  // ---- fast path: p = exp2(s), no running maximum ----
  const bool force_exact = (g.flags & PACK3D_EXACT_SOFTMAX) != 0;  // uniform
  if (!force_exact) {
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int ts = 0; ts < ntile_s; ts++) {
    const int bufi = ts & 1;
    const int m0 = ts * kTS;
    if (ts + 1 < ntile_s) load_tile(m0 + kTS);
    const bf16 *cK = sK[bufi];
    const bf16 *cV = sVt[bufi];
#pragma unroll
    for (int sub = 0; sub < kTS / 32; sub++) {
      if (m0 + 32 * sub >= g.M) break;
      f32x16 s[G];
#pragma unroll
      for (int c = 0; c < KD; c++) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8 *>(&cK[(32 * sub + rowK) * KP + 16 * c + 8 * hi]);
#pragma unroll
        for (int gi = 0; gi < G; gi++)
          s[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[gi][c], c == 0 ? zero16 : s[gi],
                                                          0, 0, 0);
      }
      if (m0 + 32 * sub + 32 > g.M) {  // past-the-end summaries take no part
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int r = (j >> 2) * 8 + hi * 4 + (j & 3);
          if (m0 + 32 * sub + swap23(r) >= g.M)
#pragma unroll
            for (int gi = 0; gi < G; gi++) s[gi][j] = -INFINITY;
        }
      }
      bf16x8 pf[G][2];
#pragma unroll
      for (int gi = 0; gi < G; gi++) {
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const float p = __builtin_amdgcn_exp2f(s[gi][j]);
          if (!ONES) lsum[gi] += p;
          pf[gi][j >> 3][j & 7] = (bf16)p;
        }
      }
#pragma unroll
      for (int t = 0; t < DT; t++) {
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(
              &cV[(32 * t + (lane & 31)) * VP + 32 * sub + 16 * c2 + 8 * hi]);
#pragma unroll
          for (int gi = 0; gi < G; gi++)
            acc[gi][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[gi][c2], acc[gi][t], 0, 0, 0);
        }
      }
    }
    if (ts + 1 < ntile_s) store_tile(bufi ^ 1);
    __syncthreads();
  }
  }

  // denominator: spare row D (lanes 0..31, register 8 of the last tile), or
  // the two half-wave partial sums. A query passes when its denominator lies
  // in [2^-100, 2^100] (far from underflow, and far enough from overflow that
  // p*v sums cannot overflow for any sane value) and every accumulator of it,
  // in both half-waves, is finite.
  constexpr float kMinDen = 7.8886091e-31f;  // 2^-100
  constexpr float kMaxDen = 1.2676506e30f;   // 2^100
  bool redo[G];
  bool any_redo = false;
#pragma unroll
  for (int gi = 0; gi < G; gi++) {
    float den;
    if (ONES)
      den = __shfl(acc[gi][DT - 1][8], lane & 31);
    else
      den = lsum[gi] + __shfl_xor(lsum[gi], 32);
    int bad = !(den >= kMinDen && den <= kMaxDen);
#pragma unroll
    for (int t = 0; t < DT; t++)
#pragma unroll
      for (int j = 0; j < 16; j++) bad |= !__builtin_isfinite(acc[gi][t][j]);
    bad |= __shfl_xor(bad, 32);
    redo[gi] = cok[gi] && (force_exact || bad);
    any_redo = any_redo || redo[gi];
    const float inv = (cok[gi] && !redo[gi]) ? 1.0f / den : 0.f;
    if (active[gi] && !redo[gi]) {
      bf16 *orow = out + (((int64_t)b * g.N + qi[gi]) * g.H + h) * D;
#pragma unroll
      for (int t = 0; t < DT; t++) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int d = 32 * t + 8 * jj + 4 * hi;
          if (d < D) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 o4;
#pragma unroll
            for (int u = 0; u < 4; u++) o4[u] = (bf16)(acc[gi][t][4 * jj + u] * inv);
            *reinterpret_cast<bf16x4 *>(orow + d) = o4;
          }
        }
      }
    }
  }
  if (!__ballot(any_redo)) return;

  // ---- exact two-pass path for the queries that failed (rare) ----
  // Reads summary fragments straight from global memory; no barriers, so
  // only the waves that need it run it.
  float mrow[G];
#pragma unroll
  for (int gi = 0; gi < G; gi++) mrow[gi] = -INFINITY;
  for (int m0 = 0; m0 < g.M; m0 += 32) {
    const bool rvalid = m0 + rowK < g.M;
    f32x16 s[G];
#pragma unroll
    for (int c = 0; c < KD; c++) {
      bf16x8 kf;
      if (rvalid)
        kf = *reinterpret_cast<const bf16x8 *>(ks + sbase + (int64_t)(m0 + rowK) * D + 16 * c + 8 * hi);
      else
#pragma unroll
        for (int x = 0; x < 8; x++) kf[x] = (bf16)0.0f;
#pragma unroll
      for (int gi = 0; gi < G; gi++)
        s[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[gi][c], c == 0 ? zero16 : s[gi], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int r = (j >> 2) * 8 + hi * 4 + (j & 3);
      if (m0 + swap23(r) < g.M)
#pragma unroll
        for (int gi = 0; gi < G; gi++) mrow[gi] = fmaxf(mrow[gi], s[gi][j]);
    }
  }
  f32x16 cneg[G];
#pragma unroll
  for (int gi = 0; gi < G; gi++) {
    mrow[gi] = fmaxf(mrow[gi], __shfl_xor(mrow[gi], 32));
#pragma unroll
    for (int j = 0; j < 16; j++) cneg[gi][j] = -mrow[gi];
#pragma unroll
    for (int t = 0; t < DT; t++)
#pragma unroll
      for (int j = 0; j < 16; j++) acc[gi][t][j] = 0.f;
    lsum[gi] = 0.f;
  }
  for (int m0 = 0; m0 < g.M; m0 += 32) {
    const bool rvalid = m0 + rowK < g.M;
    f32x16 s[G];
#pragma unroll
    for (int gi = 0; gi < G; gi++) s[gi] = cneg[gi];
#pragma unroll
    for (int c = 0; c < KD; c++) {
      bf16x8 kf;
      if (rvalid)
        kf = *reinterpret_cast<const bf16x8 *>(ks + sbase + (int64_t)(m0 + rowK) * D + 16 * c + 8 * hi);
      else
#pragma unroll
        for (int x = 0; x < 8; x++) kf[x] = (bf16)0.0f;
#pragma unroll
      for (int gi = 0; gi < G; gi++)
        s[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[gi][c], s[gi], 0, 0, 0);
    }
    bf16x8 pf[G][2];
#pragma unroll
    for (int gi = 0; gi < G; gi++) {
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int r = (j >> 2) * 8 + hi * 4 + (j & 3);
        const float p = (m0 + swap23(r) < g.M) ? __builtin_amdgcn_exp2f(s[gi][j]) : 0.f;
        if (!ONES) lsum[gi] += p;
        pf[gi][j >> 3][j & 7] = (bf16)p;
      }
    }
#pragma unroll
    for (int t = 0; t < DT; t++) {
      const int d = 32 * t + (lane & 31);
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++) {
        bf16x8 vf;
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int row = m0 + 16 * c2 + 8 * hi + e;
          vf[e] = (row < g.M && d < D) ? vs[sbase + (int64_t)row * D + d]
                                       : (bf16)((ONES && d == D) ? 1.0f : 0.0f);
        }
#pragma unroll
        for (int gi = 0; gi < G; gi++)
          acc[gi][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[gi][c2], acc[gi][t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < G; gi++) {
    float den;
    if (ONES)
      den = __shfl(acc[gi][DT - 1][8], lane & 31);
    else
      den = lsum[gi] + __shfl_xor(lsum[gi], 32);
    if (!(active[gi] && redo[gi])) continue;
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    bf16 *orow = out + (((int64_t)b * g.N + qi[gi]) * g.H + h) * D;
#pragma unroll
    for (int t = 0; t < DT; t++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int d = 32 * t + 8 * jj + 4 * hi;
        if (d < D) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 o4;
#pragma unroll
          for (int u = 0; u < 4; u++) o4[u] = (bf16)(acc[gi][t][4 * jj + u] * inv);
          *reinterpret_cast<bf16x4 *>(orow + d) = o4;
        }
      }
    }
  }
}

hipError_t launch_global_valu(const Geo &g, int dtype, const void *geom, const int32_t *coords,
                              const void *q, const void *ks, const void *vs, void *out,
                              hipStream_t s, bool *supported);

namespace {
template <int D, int G>
hipError_t run_global_mfma(const Geo &g, const void *geom, const int32_t *coords, const void *q,
                           const void *ks, const void *vs, void *out, hipStream_t s) {
  const int ntiles = (g.N + kWaves * 32 * G - 1) / (kWaves * 32 * G);
  const int64_t nwg = (int64_t)ntiles * g.B * g.H;
  hipLaunchKernelGGL((k_global_mfma<D, G>), dim3((unsigned)nwg), dim3(256), 0, s, g, geom, coords,
                     static_cast<const bf16 *>(q), static_cast<const bf16 *>(ks),
                     static_cast<const bf16 *>(vs), static_cast<bf16 *>(out), ntiles);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_global(const Geo &g, int dtype, const void *geom, const int32_t *coords,
                         const void *q, const void *ks, const void *vs, void *out, hipStream_t s,
                         bool *supported) {
  if (dtype == PACK3D_BF16 && g.excl == PACK3D_EXCL_NONE) {
    *supported = true;
    if (g.D == 48) return run_global_mfma<48, 2>(g, geom, coords, q, ks, vs, out, s);
    if (g.D == 96) return run_global_mfma<96, 1>(g, geom, coords, q, ks, vs, out, s);
  }
  return launch_global_valu(g, dtype, geom, coords, q, ks, vs, out, s, supported);
}

}  // namespace pk
