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
// of 32 that share every LDS fragment read. Summary tiles stream through
// double-buffered LDS by buffer loads straight into LDS (16 bytes per lane,
// no staging registers, no branches), one barrier per tile, the next tile in
// flight while the current one is used. Both tiles are stored chunk-major --
// a 16-byte chunk is 8 channels of one k_sum row, or one channel of 8
// consecutive v_sum rows -- laid out so that every fragment read of a
// half-wave is one contiguous 512-byte run (no bank conflicts). Per
// 32-summary sub-tile a wave computes the TRANSPOSED scores
// S^T = Ksum * Q~^T (32 summaries x 32 queries), so every lane holds 16
// scores of ONE query and the normalisation is lane-local. The k_sum rows
// are placed so that row r lands where the matrix core wants row r with bits
// 2 and 3 swapped, which makes the score registers come out exactly in the
// operand order of the next product O^T += Vsum^T * P^T: probabilities go
// from registers straight into the matrix core. The sub-tiles run as a
// three-stage software pipeline -- score products of sub-tile j+2, exp2 of
// j+1, value products of j in one step -- so that within a step no matrix
// instruction waits on a vector one and the two units overlap; each step
// also reads the next step's LDS fragments once its own have been used.
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
#include <type_traits>

#include "launch.hpp"

namespace pk {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;


__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

}  // namespace

// G = 32-query groups per wave; TS = summaries per LDS tile.
template <int D, int G, int TS>
__global__ __launch_bounds__(256, 2) void k_global_mfma(
    Geo g, const void *geom, const int32_t *__restrict__ coords, const bf16 *__restrict__ q,
    const bf16 *__restrict__ ks, const bf16 *__restrict__ vsb, bf16 *__restrict__ out,
    float *__restrict__ lse, int ntiles) {
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
  constexpr int VROWS = 64 * VPARTS;     // LDS rows per 8-summary group of a value tile
  constexpr int NKI = NCH * KPARTS, NVI = NJ8 * VPARTS;  // loads per tile
  static_assert(D % 16 == 0 && DA % 8 == 0 && (NSUB == 2 || NSUB == 4), "shape");
  static_assert(NKI % kWaves == 0 && NVI % kWaves == 0, "loads split evenly over the waves");
  // Two LDS buffers per operand, as distinct objects: the compiler can then
  // tell the in-flight loads into one buffer from the reads of the other
  // and does not wait for the loads before every read.
  __shared__ bf16x8 sK0[NCH * TS], sK1[NCH * TS];    // chunk (ch, pos): channels 8ch.., row at pos
  __shared__ bf16x8 sV0[NJ8 * VROWS], sV1[NJ8 * VROWS];  // chunk (j8, d): channel d of rows 8j8..+7

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = w % ntiles;
  const int bh = w / ntiles;
  const int h = bh % g.H, b = bh / g.H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int hi = lane >> 5;  // which half of the wave
  const int l32 = lane & 31;
  const int M32 = (g.M + 31) / 32;                       // summaries padded to Mp = 32*M32
  const int64_t bk = (int64_t)b * g.Hkv + h / g.G;         // the KV head query head h reads
  const int64_t kbase = bk * M32;                          // k_sum [B,Hkv,M32,D/8,32,8]
  const int64_t vbase = bk * M32 * 4;                      // v_sum [B,Hkv,Mp/8,D,8]
  // this KV head's summaries as two buffers (byte sizes checked on the
  // host); buffer loads keep the LDS reads countable in order, which lets
  // the fragment reads run a step ahead
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(ks + kbase * NCH * 256, M32 * NCH * 512);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vsb + vbase * D * 8, M32 * 4 * D * 16);

  // Query fragments: lane holds channels 16c + 8*hi .. +7 of its query,
  // rotated at the token's own coordinate, scaled, rounded to bf16. A token
  // whose coordinate is off the grid, or whose site went to a lower memory
  // index, takes no part (zero query, zero output row; only reachable without
  // PACK3D_VALIDATE).
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
        cok[gi] = takes_part(g, slot_map(geom, g), qi[gi], c3[0], c3[1], c3[2]);
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

  // k_sum fragments of the 32 summaries at row offset 32*pos of a k_sum tile
  auto read_k = [&](const bf16x8 *K, int pos, bf16x8 *kf) {
#pragma unroll
    for (int c = 0; c < KD; c++) kf[c] = K[(2 * c + hi) * TS + 32 * pos + l32];
  };
  // S^T = Ksum * Q~^T from k_sum fragments
  auto scores_of = [&](const bf16x8 *kf, f32x16 *s) {
#pragma unroll
    for (int c = 0; c < KD; c++)
#pragma unroll
      for (int gi = 0; gi < G; gi++)
        s[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[gi][c], c == 0 ? zero16 : s[gi], 0,
                                                        0, 0);
  };
  auto scores_from = [&](const bf16x8 *K, int pos, f32x16 *s) {
    bf16x8 kf[KD];
    read_k(K, pos, kf);
    scores_of(kf, s);
  };

  // Scores of summaries at or past M take no part (-inf); a select, so
  // whatever a stale LDS row held is discarded.
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

  // Without a spare output row the denominator is summed on the vector unit,
  // from the same bf16-rounded probabilities the value product uses (one
  // v_dot2 per pair), so the weights applied sum to one.
  bf16x2 ones2;
  ones2[0] = ones2[1] = (bf16)1.0f;
  auto sum_bf16 = [&](const bf16x8 (*pfr)[2], float *ls) {
#pragma unroll
    for (int gi = 0; gi < G; gi++)
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          bf16x2 pr2;
          pr2[0] = pfr[gi][c2][2 * e];
          pr2[1] = pfr[gi][c2][2 * e + 1];
          ls[gi] = __builtin_amdgcn_fdot2_f32_bf16(pr2, ones2, ls[gi], false);
        }
  };

  // ---- fast path: p = exp2(s), no running maximum ----
  const bool force_exact = (g.flags & PACK3D_EXACT_SOFTMAX) != 0;  // uniform
  if (!force_exact) {
    // Three-stage software pipeline over 32-summary sub-tiles: step j issues
    // the value products of sub-tile j, the exp2 of sub-tile j+1 and the
    // score products of sub-tile j+2. The 14 (D = 48) matrix instructions of
    // a step depend on none of its vector instructions, so the two streams
    // interleave freely within one wave.
    //
    // Summaries reach LDS by buffer loads straight into LDS (16 bytes per
    // lane, no staging registers), double-buffered: key tile k in buffer k&1, value
    // tile v in buffer (v+1)&1. A key tile holds the NSUB
    // sub-tiles [NSUB*k, NSUB*k + NSUB); a value tile is shifted two
    // sub-tiles back, [NSUB*v - 2, NSUB*v + NSUB - 2). Fragments are read
    // from LDS one step ahead of their products: step j reads the key
    // fragments of sub-tile j+3 and the value fragments of sub-tile j+1, so
    // both switch tiles at the same step: the step j with
    // (j + 3) % NSUB == 0 first reads key tile (j+3)/NSUB and value tile
    // (j+3)/NSUB. One barrier at the start of that step makes both visible,
    // and by then no wave reads the key and value tiles before them any
    // more, so the loads of the following tiles go into those buffers right
    // after it (NSUB steps ahead of their use).
    const int S = (g.M + 31) / 32;                 // sub-tiles with summaries
    const int IT = (S + 2 * NSUB - 1) / (2 * NSUB);  // iterations of 2*NSUB steps
    // Every lane of every load is active, so the loads need no branches:
    // lanes that would read past the summaries read the last group instead
    // (those rows are masked to -inf, or multiplied by p = 0).
    //
    // k_sum tile kt: each 64-lane load covers two 32-summary groups; within a
    // group the lane for LDS position p reads summary swap23(p), so every
    // fragment read is one contiguous 512-byte run per half-wave.
    auto issue_k = [&](int kt, bf16x8 *dK) {
#pragma unroll
      for (int r = 0; r < NKI / kWaves; r++) {
        const int i = wv + kWaves * r;
        const int ch = i / KPARTS, part = i % KPARTS;
        const int g32 = min(kt * NSUB + 2 * part + hi, M32 - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (lds_ptr)&dK[ch * TS + part * 64], 16,
            (uint32_t)(((g32 * NCH + ch) * 32 + swap23(l32)) * 16), 0, 0, 0);
      }
    };
    // v_sum tile vt: LDS chunk (j8, d) = channel d of summaries 8*j8.. of the
    // tile. Only rows d < D are loaded (the lanes of the other rows are
    // masked off). Rows D.. of both buffers are written once, below, and
    // never overwritten: all zeros, except row D when it carries the
    // denominator (bf16 ones), so the padding output rows stay finite and
    // the spare row sums the weights.
    static_assert(!ONES || VPARTS == 1, "the denominator row is in the first part");
    auto issue_v = [&](int vt, bf16x8 *dV) {
      const int g8base = 4 * (vt * NSUB - 2);
#pragma unroll
      for (int r = 0; r < NVI / kWaves; r++) {
        const int i = wv + kWaves * r;
        const int j8 = i / VPARTS, part = i % VPARTS;
        const int d = part * 64 + lane;
        const int g8 = min(max(g8base + j8, 0), 4 * M32 - 1);
        if (part * 64 + 64 <= D || d < D)  // the first test is known at compile time
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)&dV[j8 * VROWS + part * 64], 16,
                                                   (uint32_t)((g8 * D + d) * 16), 0, 0, 0);
      }
    };
    {
      constexpr int NCR = VROWS - D;  // constant rows per 8-summary group
      for (int e = threadIdx.x; e < 2 * NJ8 * NCR; e += 256) {
        const int buf = e / (NJ8 * NCR), j8 = (e / NCR) % NJ8, row = D + e % NCR;
        bf16x8 c;
#pragma unroll
        for (int u = 0; u < 8; u++) c[u] = (bf16)((ONES && row == D) ? 1.0f : 0.0f);
        (buf ? sV1 : sV0)[j8 * VROWS + row] = c;
      }
    }

    issue_k(0, sK0);
    issue_v(0, sV1);  // sub-tiles -2 .. NSUB-3 (only 0, 1 exist for NSUB = 4)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue_k(1, sK1);
    issue_v(1, sV0);

    f32x16 s[2][G];        // scores of sub-tiles j+1, j+2 (by parity)
    bf16x8 pf[2][G][2];    // probabilities of sub-tiles j, j+1 (by parity)
    bf16x8 kf[KD];         // key fragments of sub-tile j+2
    bf16x8 vf[DT][2];      // value fragments of sub-tile j
    // value fragments of sub-tile j at position pos of a value tile
    auto read_v = [&](const bf16x8 *V, int pos) {
#pragma unroll
      for (int t = 0; t < DT; t++)
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++) vf[t][c2] = V[(4 * pos + 2 * c2 + hi) * VROWS + 32 * t + l32];
    };
    scores_from(sK0, 0, s[0]);
    mask_tail(s[0], 0);
    scores_from(sK0, 1, s[1]);
#pragma unroll
    for (int gi = 0; gi < G; gi++)
#pragma unroll
      for (int j = 0; j < 16; j++) pf[0][gi][j >> 3][j & 7] = (bf16)__builtin_amdgcn_exp2f(s[0][gi][j]);
    if constexpr (!ONES) sum_bf16(pf[0], lsum);
    // The prologue is step -1: it reads key sub-tile 2 and value sub-tile 0,
    // both in tile 2/NSUB. With two sub-tiles per tile that is tile 1, so
    // this is a tile-switch step like the ones in the loop.
    if constexpr (NSUB == 2) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      issue_k(2, sK0);
      issue_v(2, sV1);
      read_k(sK1, 0, kf);
      read_v(sV0, 0);
    } else {
      read_k(sK0, 2, kf);  // key tile 0
      read_v(sV1, 2);      // value tile 0, which starts at sub-tile -2
    }

    // one step; JJ = position in the 2*NSUB-step iteration (compile time)
    auto step = [&](int it, auto jc, auto mc) {
      constexpr int JJ = decltype(jc)::value;
      constexpr bool MASK = decltype(mc)::value;  // some summary of sub-tile j+1 may be past M
      constexpr int KT = (JJ + 3) / NSUB;  // key tile of sub-tile j+3, from 2*it
      constexpr int KB = KT & 1;
      constexpr int VB = (KT + 1) & 1;     // value tile of sub-tile j+1: 2*it + KT
      constexpr int POS = (JJ + 3) % NSUB;
      constexpr int P = JJ & 1;
      const bf16x8 *nK = KB ? sK1 : sK0;
      bf16x8 *nV = VB ? sV1 : sV0;
      const int j = 2 * NSUB * it + JJ;
      // each step is its own scheduling region: the compiler may not pull the
      // next step's exp2 of the scores just issued into this one, where it
      // would wait for those products to drain
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (POS == 0) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads landed, LDS reads done
        __syncthreads();
        issue_k(2 * it + KT + 1, KB ? sK0 : sK1);
        issue_v(2 * it + KT + 1, KB ? sV1 : sV0);
      }
      if constexpr (MASK) mask_tail(s[P ^ 1], 32 * (j + 1));
      scores_of(kf, s[P]);  // sub-tile j+2
      read_k(nK, POS, kf);  // sub-tile j+3, for the next step
#pragma unroll
      for (int gi = 0; gi < G; gi++)
#pragma unroll
        for (int jr = 0; jr < 16; jr++)
          pf[P ^ 1][gi][jr >> 3][jr & 7] = (bf16)__builtin_amdgcn_exp2f(s[P ^ 1][gi][jr]);
      if constexpr (!ONES) sum_bf16(pf[P ^ 1], lsum);
#pragma unroll
      for (int gi = 0; gi < G; gi++)
#pragma unroll
        for (int t = 0; t < DT; t++)
#pragma unroll
          for (int c2 = 0; c2 < 2; c2++)
            acc[gi][t] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t][c2], pf[P][gi][c2], acc[gi][t], 0, 0, 0);
      read_v(nV, POS);  // sub-tile j+1, for the next step
      __builtin_amdgcn_sched_barrier(0);
    };
    // Iterations before IT_CLEAN only see sub-tiles that lie wholly below M,
    // so their steps carry no mask (and no branch that would split a step's
    // matrix and vector streams); the last iteration(s) mask.
    const int IT_CLEAN = min(IT, max(0, (g.M / 32 - 1) / (2 * NSUB)));
    auto iteration = [&](int it, auto mc) {
      step(it, std::integral_constant<int, 0>{}, mc);
      step(it, std::integral_constant<int, 1>{}, mc);
      step(it, std::integral_constant<int, 2>{}, mc);
      step(it, std::integral_constant<int, 3>{}, mc);
      if constexpr (NSUB == 4) {
        step(it, std::integral_constant<int, 4>{}, mc);
        step(it, std::integral_constant<int, 5>{}, mc);
        step(it, std::integral_constant<int, 6>{}, mc);
        step(it, std::integral_constant<int, 7>{}, mc);
      }
    };
    int it = 0;
    for (; it < IT_CLEAN; it++) iteration(it, std::false_type{});
    for (; it < IT; it++) iteration(it, std::true_type{});
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
    if (active[gi] && !redo[gi]) {
      store_rows(gi, cok[gi] ? 1.0f / den : 0.f);
      // scores were not shifted: the log-sum-exp is log2 of the denominator
      if (lse && hi == 0) lse[((int64_t)b * g.N + qi[gi]) * g.H + h] = cok[gi] ? __log2f(den) : -INFINITY;
    }
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
        pf[gi][j >> 3][j & 7] = (bf16)p;
      }
    }
    if constexpr (!ONES) sum_bf16(pf, lsum);
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
    if (active[gi] && redo[gi]) {
      store_rows(gi, den > 0.f ? 1.0f / den : 0.f);
      if (lse && hi == 0)
        lse[((int64_t)b * g.N + qi[gi]) * g.H + h] = den > 0.f ? mrow[gi] + __log2f(den) : -INFINITY;
    }
  }
}

hipError_t launch_global_valu(const Geo &g, int dtype, const void *geom, const int32_t *coords,
                              const void *q, const void *ks, const void *vs, void *out,
                              float *lse, hipStream_t s, bool *supported);

namespace {
template <int D, int G, int TS>
hipError_t run_global_mfma(const Geo &g, const void *geom, const int32_t *coords, const void *q,
                           const void *ks, const void *vs, void *out, float *lse, hipStream_t s) {
  const int ntiles = (g.N + kWaves * 32 * G - 1) / (kWaves * 32 * G);
  const int64_t nwg = (int64_t)ntiles * g.B * g.H;
  hipLaunchKernelGGL((k_global_mfma<D, G, TS>), dim3((unsigned)nwg), dim3(256), 0, s, g, geom, coords,
                     static_cast<const bf16 *>(q), static_cast<const bf16 *>(ks),
                     static_cast<const bf16 *>(vs), static_cast<bf16 *>(out), lse, ntiles);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_global(const Geo &g, int dtype, const void *geom, const int32_t *coords,
                         const void *q, const void *ks, const void *vs, void *out, float *lse,
                         hipStream_t s, bool *supported) {
  // the matrix-core path addresses one KV head's summaries with 32-bit byte
  // offsets
  const int64_t head_bytes = (int64_t)((g.M + 31) / 32) * 32 * g.D * 2;
  if (dtype == PACK3D_BF16 && g.excl == PACK3D_EXCL_NONE && head_bytes <= INT32_MAX) {
    *supported = true;
    if (g.D == 48) return run_global_mfma<48, 2, 128>(g, geom, coords, q, ks, vs, out, lse, s);
    if (g.D == 96) return run_global_mfma<96, 1, 64>(g, geom, coords, q, ks, vs, out, lse, s);
  }
  return launch_global_valu(g, dtype, geom, coords, q, ks, vs, out, lse, s, supported);
}

}  // namespace pk
