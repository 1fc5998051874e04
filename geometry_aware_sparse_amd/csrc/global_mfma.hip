// Query-to-summary attention on bf16 matrix cores (Geometry Matters in Packed
// 3D Attention, project page Ch. 3, Contract 2; paper summary §3.5, §B.10).
//
// The global branch is a dense contraction -- every query against all M
// summaries -- so it runs as a flash-style loop on v_mfma_f32_32x32x16_bf16
// with an fp32 online softmax and never forms the token x summary score
// matrix (paper summary §3.5).
//
// Layout of the work. A workgroup of 4 waves owns 64*G*4 consecutive tokens
// (packed order) of one (batch, head); a wave owns 32*G of them as G groups
// of 32 that share every LDS fragment read. Summary tiles of TS rows stream
// through double-buffered LDS by direct global->LDS loads (16 bytes per
// lane, no staging registers): the next tile is in flight while the current
// one is used, one barrier per tile. Both tiles are stored chunk-major -- a
// 16-byte chunk is 8 channels of one k_sum row, or one channel of 8
// consecutive v_sum rows -- laid out so that every fragment read of a
// half-wave is one contiguous 512-byte run (no bank conflicts). Per
// 32-summary sub-tile a wave computes the TRANSPOSED scores
// S^T = Ksum * Q~^T (32 summaries x 32 queries), so every lane holds 16
// scores of ONE query and the normalisation is lane-local. The k_sum rows
// are placed so that row r lands where the matrix core wants row r with bits
// 2 and 3 swapped, which makes the score registers come out exactly in the
// operand order of the next product O^T += Vsum^T * P^T: probabilities go
// from registers straight into the matrix core. The products of sub-tile
// n+1 are issued before the exponentials of sub-tile n so that the matrix
// core and the vector unit overlap within one wave.
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
constexpr int kWaves = 4;

__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
typedef __attribute__((address_space(3))) void *lds_ptr;

// Scheduling hint for one sub-tile body: alternate one matrix instruction
// with four vector instructions so that a wave keeps issuing exp2/convert
// work while its own products run (a wave issues in order; a run of matrix
// instructions would otherwise stall it on the busy matrix pipe).
#define SCHED_INTERLEAVE()                                        \
  do {                                                            \
    _Pragma("unroll") for (int _i = 0; _i < 14; _i++) {           \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          \
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);          \
    }                                                             \
  } while (0)
}  // namespace

// G = 32-query groups per wave; TS = summaries per LDS tile.
template <int D, int G, int TS>
__global__ __launch_bounds__(256, 2) void k_global_mfma(
    Geo g, const void *geom, const int32_t *__restrict__ coords, const bf16 *__restrict__ q,
    const bf16 *__restrict__ ks, const bf16 *__restrict__ vsb, bf16 *__restrict__ out,
    int ntiles) {
  constexpr int DA = D / 3;
  constexpr int KD = D / 16;             // 16-deep steps of Ksum * Q~^T
  constexpr bool ONES = (D % 32) != 0;   // spare output rows carry the denominator
  constexpr int DT = (D + 31) / 32;      // 32-row tiles of O^T
  constexpr int DPAD = DT * 32;
  constexpr int QPW = 32 * G;            // queries per wave
  constexpr int NCH = D / 8;             // 16-byte chunks per k_sum row
  constexpr int NJ8 = TS / 8;            // groups of 8 summaries per tile
  constexpr int NSUB = TS / 32;
  constexpr int KPARTS = TS / 64;        // 64-lane loads per k_sum chunk row
  constexpr int VPARTS = (DPAD + 63) / 64;
  constexpr int NKI = NCH * KPARTS, NVI = NJ8 * VPARTS;  // loads per tile
  static_assert(D % 16 == 0 && DA % 8 == 0 && TS % 64 == 0, "shape");
  // Two LDS buffers per operand, as distinct objects: the compiler can then
  // tell the in-flight global->LDS loads into one buffer from the reads of
  // the other and does not wait for the loads before every read.
  __shared__ bf16x8 sK0[NCH * TS], sK1[NCH * TS];    // chunk (ch, pos): channels 8ch.., row at pos
  __shared__ bf16x8 sV0[NJ8 * DPAD], sV1[NJ8 * DPAD];  // chunk (j8, d): channel d of rows 8j8..+7

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = w % ntiles;
  const int bh = w / ntiles;
  const int h = bh % g.H, b = bh / g.H;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int hi = lane >> 5;  // which half of the wave
  const int l32 = lane & 31;
  const int M32 = (g.M + 31) / 32;                       // summaries padded to Mp = 32*M32
  const int64_t kbase = ((int64_t)b * g.H + h) * M32;      // k_sum [B,H,M32,D/8,32,8]
  const int64_t vbase = ((int64_t)b * g.H + h) * M32 * 4;  // v_sum [B,H,Mp/8,D,8]

  // value tiles start as zeros (rows past M are never loaded and must stay
  // finite), with the all-ones spare row that yields the denominator
  for (int e = threadIdx.x; e < NJ8 * DPAD; e += 256) {
    const int d = e % DPAD;
    bf16x8 c;
#pragma unroll
    for (int x = 0; x < 8; x++) c[x] = (bf16)((ONES && d == D) ? 1.0f : 0.0f);
    sV0[e] = c;
    sV1[e] = c;
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
      qi[gi] = tile * (kWaves * QPW) + wv * QPW + gi * 32 + l32;
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

  // Direct global->LDS loads of tile ts into buffer bb: each 64-lane load
  // writes 64 consecutive chunks; lanes whose row lies past M stay idle.
  auto issue_tile = [&](int ts, bf16x8 *dK, bf16x8 *dV) {
    const int m0 = ts * TS;
    for (int i = wv; i < NKI + NVI; i += kWaves) {
      if (i < NKI) {
        // 64 lanes = two 32-summary groups; within a group the lane for LDS
        // position p reads summary swap23(p): 512 contiguous bytes per half
        const int ch = i / KPARTS, part = i % KPARTS;
        const int g32 = m0 / 32 + 2 * part + hi;
        if (g32 < M32)
          __builtin_amdgcn_global_load_lds(
              ks + (((kbase + g32) * NCH + ch) * 32 + swap23(l32)) * 8,
              (lds_ptr)&dK[ch * TS + part * 64], 16, 0, 0);
      } else {
        const int iv = i - NKI;
        const int j8 = iv / VPARTS, part = iv % VPARTS;
        const int d = part * 64 + lane;
        const int g8 = m0 / 8 + j8;
        if (d < D && g8 < 4 * M32)
          __builtin_amdgcn_global_load_lds(vsb + ((vbase + g8) * D + d) * 8,
                                           (lds_ptr)&dV[j8 * DPAD + part * 64], 16, 0, 0);
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
  const int ntile_s = (g.M + TS - 1) / TS;

  // S^T = Ksum * Q~^T from the k_sum fragments of one sub-tile
  auto scores_from = [&](const bf16x8 *kf, f32x16 *s) {
#pragma unroll
    for (int c = 0; c < KD; c++)
#pragma unroll
      for (int gi = 0; gi < G; gi++)
        s[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[gi][c], c == 0 ? zero16 : s[gi], 0,
                                                        0, 0);
  };

  // Scores of summaries past M take no part (-inf). Applied when a sub-tile's
  // scores are handed over, outside the block that overlaps the next
  // products with this sub-tile's exp2, so that block has no branch in it.
  auto mask_tail = [&](f32x16 *s, int mbase) {
    if (mbase + 32 > g.M) {
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int r = (j >> 2) * 8 + hi * 4 + (j & 3);
        if (mbase + swap23(r) >= g.M)
#pragma unroll
          for (int gi = 0; gi < G; gi++) s[gi][j] = -INFINITY;
      }
    }
  };

  // ---- fast path: p = exp2(s), no running maximum ----
  const bool force_exact = (g.flags & PACK3D_EXACT_SOFTMAX) != 0;  // uniform
  if (!force_exact) {
    __syncthreads();  // value tiles initialised before any load lands
    issue_tile(0, sK0, sV0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Software pipeline over 32-summary sub-tiles: at sub-tile n the
    // products of n+1 (fragments read one step ahead) and the value
    // fragments of n are issued first, then the exp2 of n runs while the
    // matrix core works, then the value products of n. At the last sub-tile
    // of an LDS tile the barrier comes before the exp2, so the first products
    // of the next tile overlap it too; every read of the old buffer has
    // landed in registers before that barrier, after which the other waves
    // may refill it.
    bf16x8 kf[2][KD];
    f32x16 s_cur[G], s_nxt[G];
#pragma unroll
    for (int c = 0; c < KD; c++) kf[0][c] = sK0[(2 * c + hi) * TS + l32];
    scores_from(kf[0], s_cur);
    mask_tail(s_cur, 0);
    if (NSUB > 1) {
#pragma unroll
      for (int c = 0; c < KD; c++) kf[1][c] = sK0[(2 * c + hi) * TS + 32 + l32];
    }
    auto run_tile = [&](int ts, const bf16x8 *cK, const bf16x8 *cV, bf16x8 *nK, bf16x8 *nV) {
      const int m0 = ts * TS;
      const bool more = ts + 1 < ntile_s;  // uniform; then this tile is full
      if (more) issue_tile(ts + 1, nK, nV);
#pragma unroll
      for (int sub = 0; sub < NSUB; sub++) {
        if (m0 + 32 * sub >= g.M) break;
        const bool last = sub == NSUB - 1;
        bf16x8 vf[DT][2];
#pragma unroll
        for (int t = 0; t < DT; t++)
#pragma unroll
          for (int c2 = 0; c2 < 2; c2++) vf[t][c2] = cV[(4 * sub + 2 * c2 + hi) * DPAD + 32 * t + l32];
        if (!last) {
          scores_from(kf[(sub + 1) & 1], s_nxt);
          if (sub + 2 < NSUB) {
#pragma unroll
            for (int c = 0; c < KD; c++) kf[sub & 1][c] = cK[(2 * c + hi) * TS + 32 * (sub + 2) + l32];
          }
        } else if (more) {
          __builtin_amdgcn_s_waitcnt(0);  // next tile landed, old-buffer reads done
          __syncthreads();
#pragma unroll
          for (int c = 0; c < KD; c++) kf[0][c] = nK[(2 * c + hi) * TS + l32];
          scores_from(kf[0], s_nxt);
          if (NSUB > 1) {
#pragma unroll
            for (int c = 0; c < KD; c++) kf[1][c] = nK[(2 * c + hi) * TS + 32 + l32];
          }
        }
        bf16x8 pf[G][2];
#pragma unroll
        for (int gi = 0; gi < G; gi++) {
#pragma unroll
          for (int j = 0; j < 16; j++) {
            const float p = __builtin_amdgcn_exp2f(s_cur[gi][j]);
            if (!ONES) lsum[gi] += p;
            pf[gi][j >> 3][j & 7] = (bf16)p;
          }
        }
#pragma unroll
        for (int gi = 0; gi < G; gi++)
#pragma unroll
          for (int t = 0; t < DT; t++)
#pragma unroll
            for (int c2 = 0; c2 < 2; c2++)
              acc[gi][t] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t][c2], pf[gi][c2], acc[gi][t], 0, 0, 0);
        SCHED_INTERLEAVE();
#pragma unroll
        for (int gi = 0; gi < G; gi++) s_cur[gi] = s_nxt[gi];
        mask_tail(s_cur, last ? m0 + TS : m0 + 32 * (sub + 1));
      }
    };
    for (int ts = 0; ts < ntile_s; ts += 2) {
      run_tile(ts, sK0, sV0, sK1, sV1);
      if (ts + 1 < ntile_s) run_tile(ts + 1, sK1, sV1, sK0, sV0);
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
  auto store_rows = [&](int gi, float inv) {
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
  };
#pragma unroll
  for (int gi = 0; gi < G; gi++) {
    float den;
    if (ONES)
      den = __shfl(acc[gi][DT - 1][8], l32);
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
    if (active[gi] && !redo[gi]) store_rows(gi, cok[gi] ? 1.0f / den : 0.f);
  }
  if (!__ballot(any_redo)) return;

  // ---- exact two-pass path for the queries that failed (rare) ----
  // Reads summary fragments straight from global memory; no barriers, so
  // only the waves that need it run it.
  const int rowK = swap23(l32);
  auto kfrag = [&](int m0, int c) {  // m0: multiple of 32, inside the padded range
    return *reinterpret_cast<const bf16x8 *>(
        ks + (((kbase + m0 / 32) * NCH + 2 * c + hi) * 32 + rowK) * 8);
  };
  float mrow[G];
#pragma unroll
  for (int gi = 0; gi < G; gi++) mrow[gi] = -INFINITY;
  for (int m0 = 0; m0 < g.M; m0 += 32) {
    f32x16 s[G];
#pragma unroll
    for (int c = 0; c < KD; c++) {
      const bf16x8 kf = kfrag(m0, c);
#pragma unroll
      for (int gi = 0; gi < G; gi++)
        s[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[gi][c], c == 0 ? zero16 : s[gi], 0,
                                                        0, 0);
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
    f32x16 s[G];
#pragma unroll
    for (int gi = 0; gi < G; gi++) s[gi] = cneg[gi];
#pragma unroll
    for (int c = 0; c < KD; c++) {
      const bf16x8 kf = kfrag(m0, c);
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
      const int d = 32 * t + l32;
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++) {
        const int g8 = (m0 + 16 * c2 + 8 * hi) / 8;
        bf16x8 vf;
        if (d < D) {
          vf = *reinterpret_cast<const bf16x8 *>(vsb + ((vbase + g8) * D + d) * 8);
        } else {
#pragma unroll
          for (int x = 0; x < 8; x++) vf[x] = (bf16)((ONES && d == D) ? 1.0f : 0.0f);
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
      den = __shfl(acc[gi][DT - 1][8], l32);
    else
      den = lsum[gi] + __shfl_xor(lsum[gi], 32);
    if (active[gi] && redo[gi]) store_rows(gi, den > 0.f ? 1.0f / den : 0.f);
  }
}

hipError_t launch_global_valu(const Geo &g, int dtype, const void *geom, const int32_t *coords,
                              const void *q, const void *ks, const void *vs, void *out,
                              hipStream_t s, bool *supported);

namespace {
template <int D, int G, int TS>
hipError_t run_global_mfma(const Geo &g, const void *geom, const int32_t *coords, const void *q,
                           const void *ks, const void *vs, void *out, hipStream_t s) {
  const int ntiles = (g.N + kWaves * 32 * G - 1) / (kWaves * 32 * G);
  const int64_t nwg = (int64_t)ntiles * g.B * g.H;
  hipLaunchKernelGGL((k_global_mfma<D, G, TS>), dim3((unsigned)nwg), dim3(256), 0, s, g, geom, coords,
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
    if (g.D == 48) return run_global_mfma<48, 2, 128>(g, geom, coords, q, ks, vs, out, s);
    if (g.D == 96) return run_global_mfma<96, 1, 64>(g, geom, coords, q, ks, vs, out, s);
  }
  return launch_global_valu(g, dtype, geom, coords, q, ks, vs, out, s, supported);
}

}  // namespace pk
