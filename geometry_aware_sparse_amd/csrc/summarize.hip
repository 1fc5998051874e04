// Rotate-then-pool block summaries (Geometry Matters in Packed 3D Attention,
// project page Ch. 3 "Rotate first, then pool"; paper summary §3.2, §B.5),
// and the summary-centre variant under PACK3D_SUMMARY_CENTRE (paper summary
// §B.7, §B.8): the mean of the unrotated keys, rotated once at the block
// centre.
//
// One workgroup per (group of 8 consecutive summaries, batch); the summary
// count is padded to Mp = 32*ceil(M/32) and padding slots are written as 0.
// The workgroup stages the members' memory positions (slot map lookups in
// canonical within-block-slot order) in LDS; a thread owns one block of the
// group and one chunk of CW channels of the token's contiguous [H, D] row,
// and accumulates the members in fp32 in that order -- so the summaries are
// the same bits under any packing of the tokens. HBM-bound: every K and V
// element is read once, with 16-byte loads.
//
// Outputs, both blocked so that the matrix-core kernel streams them with
// contiguous 16-byte-per-lane loads:
//   k_sum [B, H, Mp/32, Dp/8, 32, 8]: element (m, d) at [b, h, m/32, d/8, m%32, d%8]
//                                   (Dp = 8*ceil(D/8); padding channels are 0)
//   v_sum [B, H, Mp/8, D, 8]:        element (m, d) at [b, h, m/8, d, m%8]
// The v_sum means pass through LDS so that each (channel, group) is written
// as one 16-byte chunk.
#include "launch.hpp"

namespace pk {

constexpr int kMaxMembers = 512;  // member slots staged in LDS per pass (8 blocks)

// Summary-centre variant: rotate the (unrotated) mean key of block m, a chunk
// of CW channels of axis a starting at plane p0, at the block centre
// origin + (extent - 1) / 2, the extent clipped at the grid edge. An odd
// extent puts the centre on a grid coordinate, origin + l, whose (cos, sin)
// is a table row; an even one puts it at origin + l + 1/2, whose (cos, sin)
// follow from row l and the table's half-angle row by the angle-addition
// formulas. cs_at(l, p) gives plane p's (cos, sin) at local coordinate l.
template <int CW, typename CsAt>
__device__ __forceinline__ void rotate_at_centre(const Geo &g, int m, int a, int p0,
                                                 const float2 *tab, CsAt cs_at, float *x) {
  const int mz = m / (g.My * g.Mx), my = (m / g.Mx) % g.My, mx = m % g.Mx;
  const int o = a == 0 ? mz * g.bz : (a == 1 ? my * g.by : mx * g.bx);
  const int ext = min(a == 0 ? g.bz : (a == 1 ? g.by : g.bx), (a == 0 ? g.Z : (a == 1 ? g.Y : g.X)) - o);
  const int l = (ext - 1) / 2;
  const bool odd = (ext & 1) != 0;
#pragma unroll
  for (int u = 0; u < CW; u += 2) {
    const int p = p0 + u / 2;
    float2 t = cs_at(l, p);
    if (!odd) {
      const float2 hh = rope_half(tab, g, p);
      t = make_float2(t.x * hh.x - t.y * hh.y, t.y * hh.x + t.x * hh.y);
    }
    rotate(x[u], x[u + 1], t);
  }
}

template <typename T, int CW, bool CENTRE>
__global__ __launch_bounds__(512) void k_summarize(Geo g, const void *geom, const T *k,
                                                   const T *v, T *ks, T *vsb) {
  __shared__ int s_slot[kMaxMembers];
  extern __shared__ float s_vt[];  // [H*D][8] value means for the transposed write
  const int g8 = blockIdx.x, b = blockIdx.y;
  const int Mp = (g.M + 31) / 32 * 32;
  const int Dp = (g.D + 7) / 8 * 8;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int da = g.D / 3;
  const int NC = g.Hkv * g.D / CW;        // channel chunks per token row
  const int CPT = blockDim.x / 8;       // chunk lanes per block
  const int s = threadIdx.x / CPT;      // block of the group owned by this thread
  const int c0 = threadIdx.x % CPT;
  const int m = 8 * g8 + s;
  const int mz = m / (g.My * g.Mx), my = (m / g.Mx) % g.My, mx = m % g.Mx;
  const int o3[3] = {mz * g.bz, my * g.by, mx * g.bx};
  const int64_t bh0 = (int64_t)b * g.Hkv;

  // members of all 8 blocks, in passes of kMaxMembers / 8 per block
  const int per = kMaxMembers / 8;
  // every thread runs the same number of rounds (the barriers below need it)
  const int rounds = (NC + CPT - 1) / CPT;  // usually 1
  for (int rd = 0; rd < rounds; rd++) {
    const int c = c0 + rd * CPT;
    const bool act = c < NC;
    const int h = act ? (c * CW) / g.D : 0, d0 = act ? (c * CW) % g.D : 0;
    float ka[CW], va[CW];
#pragma unroll
    for (int u = 0; u < CW; u++) ka[u] = va[u] = 0.f;
    int cnt = 0;
    for (int r0 = 0; r0 < g.vol; r0 += per) {
      const int nr = min(per, g.vol - r0);
      __syncthreads();
      for (int e = threadIdx.x; e < 8 * nr; e += blockDim.x) {
        const int ss = e / nr, rr = r0 + e % nr, mm = 8 * g8 + ss;
        int j = -1;
        if (mm < g.M) {
          const int z = (mm / (g.My * g.Mx)) * g.bz + rr / (g.by * g.bx);
          const int y = ((mm / g.Mx) % g.My) * g.by + (rr / g.bx) % g.by;
          const int x = (mm % g.Mx) * g.bx + rr % g.bx;
          if (z < g.Z && y < g.Y && x < g.X) j = slot_get(g, slot, site_of(g, z, y, x));
        }
        s_slot[e] = j;
      }
      __syncthreads();
#pragma unroll 4
      for (int r = 0; r < nr; r++) {
        const int j = s_slot[s * nr + r];
        if (j < 0 || !act) continue;
        cnt++;
        const int rr = r0 + r;
        const int c3[3] = {o3[0] + rr / (g.by * g.bx), o3[1] + (rr / g.bx) % g.by, o3[2] + rr % g.bx};
        const int64_t off = (((int64_t)b * g.N + j) * g.Hkv + h) * g.D + d0;
        float kx[CW], vx[CW];
        if constexpr (CW == 8 && sizeof(T) == 2) {
          const bf16x8 kr = *reinterpret_cast<const bf16x8 *>(k + off);
          const bf16x8 vr = *reinterpret_cast<const bf16x8 *>(v + off);
#pragma unroll
          for (int u = 0; u < 8; u++) {
            kx[u] = (float)kr[u];
            vx[u] = (float)vr[u];
          }
        } else {
#pragma unroll
          for (int u = 0; u < CW; u++) {
            kx[u] = to_f32(k[off + u]);
            vx[u] = to_f32(v[off + u]);
          }
        }
        if constexpr (!CENTRE) {
#pragma unroll
          for (int u = 0; u < CW; u += 2) {
            const int dd = d0 + u, a = dd / da;
            rotate(kx[u], kx[u + 1], rope_cs(tab, g, a, c3[a], (dd % da) / 2));
          }
        }
#pragma unroll
        for (int u = 0; u < CW; u++) {
          ka[u] += kx[u];
          va[u] += vx[u];
        }
      }
    }
    if (!act) continue;
    // mean = sum / count (a division, as in the definition); empty -> 0
    float km[CW];
#pragma unroll
    for (int u = 0; u < CW; u++) km[u] = cnt > 0 ? ka[u] / (float)cnt : 0.0f;
    if (CENTRE && m < g.M) {  // padding slots stay 0 (and have no extent)
      const int a = d0 / da;  // a chunk lies within one axis
      rotate_at_centre<CW>(g, m, a, (d0 % da) / 2, tab,
                           [&](int l, int p) { return rope_cs(tab, g, a, o3[a] + l, p); }, km);
    }
    const int64_t ko = ((((bh0 + h) * (Mp / 32) + m / 32) * (Dp / 8) + d0 / 8) * 32 + m % 32) * 8;
#pragma unroll
    for (int u = 0; u < CW; u++) {
      ks[ko + (d0 + u) % 8] = from_f32<T>(km[u]);
      s_vt[(h * g.D + d0 + u) * 8 + s] = cnt > 0 ? va[u] / (float)cnt : 0.0f;
    }
  }
  __syncthreads();
  // v_sum: one 16-byte (bf16) chunk per (head, channel)
  for (int e = threadIdx.x; e < g.Hkv * g.D; e += blockDim.x) {
    const int h = e / g.D, d = e % g.D;
    T *dst = vsb + (((bh0 + h) * (Mp / 8) + g8) * g.D + d) * 8;
#pragma unroll
    for (int u = 0; u < 8; u++) dst[u] = from_f32<T>(s_vt[e * 8 + u]);
  }
  // padding channels D..Dp of k_sum are zero
  for (int e = threadIdx.x; e < 8 * g.Hkv * (Dp - g.D); e += blockDim.x) {
    const int ss = e / (g.Hkv * (Dp - g.D)), rem = e % (g.Hkv * (Dp - g.D));
    const int h = rem / (Dp - g.D), d = g.D + rem % (Dp - g.D), mm = 8 * g8 + ss;
    ks[((((bh0 + h) * (Mp / 32) + mm / 32) * (Dp / 8) + d / 8) * 32 + mm % 32) * 8 + d % 8] =
        from_f32<T>(0.0f);
  }
}

// bf16 rows whose head dim is a multiple of 8: the same summaries (same
// members, same order, fp32 sums; the rotation is folded into the sums'
// fused multiply-adds, so the last bits may differ from k_summarize),
// arranged so that memory latency is paid a few times per workgroup instead
// of once per member.
//   1. The members' slots and the RoPE rows of the 8 blocks' coordinate
//      ranges are staged in LDS (one round of loads, one barrier).
//   2. A thread owns one block and one 16-byte chunk of the token row; it
//      issues the K and V loads of kBatch members at once, then adds them
//      up in within-block-slot order: keys through fused multiply-adds with
//      their (cos, sin), values through v_dot2 with weights (1, 0), (0, 1).
//      A member that is absent reads a zero chunk of the geometry buffer
//      instead, so it contributes exact zeros with no select.
//   3. The means take one reciprocal per block and a residual correction.
//   4. The value means are transposed through LDS with an odd row pitch, so
//      the writes of a wave fall in distinct banks.
// Members whose loads are in flight together. Four, with five waves per
// SIMD asked of the compiler (93 VGPRs): three 6-wave workgroups share a CU
// instead of two, and the 65,536-token volume's pass takes 24.7 us instead
// of 29.0 us with eight members at 122 VGPRs.
constexpr int kBatch = 4;

template <bool CENTRE>
__global__ __launch_bounds__(512, 5) void k_summarize_b8(Geo g, const void *geom, const bf16 *k,
                                                       const bf16 *v, bf16 *ks, bf16 *vsb,
                                                       int nrow) {
  extern __shared__ float s_dyn[];
  const int NC = g.Hkv * g.D / 8;          // 16-byte chunks per token row
  const int NT = 8 * NC;
  const int per = min(g.vol, kMaxMembers / 8);  // members staged per pass and block
  const int P = g.P;
  int *s_slot = reinterpret_cast<int *>(s_dyn);                  // [8][per]
  int *s_lc = s_slot + 8 * per;                                  // [per] packed (lz, ly, lx)
  float2 *s_cs = reinterpret_cast<float2 *>(s_dyn + 8 * per + per + ((9 * per) & 1));  // [8][nrow][P]
  float *s_vt = reinterpret_cast<float *>(s_cs + 8 * nrow * P);  // [8][NC][9]
  const int g8 = blockIdx.x, b = blockIdx.y;
  const int Mp = (g.M + 31) / 32 * 32;
  const int32_t *slot = slot_map(geom, g);
  const float2 *tab = rope_table(geom, g);
  const int s = threadIdx.x / NC;        // block of the group owned by this thread
  const int c = threadIdx.x - s * NC;    // chunk of the token row
  const int h = (c * 8) / g.D, d0 = c * 8 - h * g.D;
  const int DA = g.D / 3;
  const int a = d0 / DA, p0 = (d0 - a * DA) / 2;
  const int m = 8 * g8 + s;
  // origin of block 8*g8 + ss (block-raster order), for every ss, computed
  // from the group's first block once (wave-uniform)
  const int m0 = 8 * g8;
  const int MyMx = g.My * g.Mx;
  int oz[8], oy[8], ox[8];
  {
    int mz = m0 / MyMx, rem = m0 - mz * MyMx;
    int my = rem / g.Mx, mx = rem - my * g.Mx;
#pragma unroll
    for (int ss = 0; ss < 8; ss++) {
      oz[ss] = mz * g.bz;
      oy[ss] = my * g.by;
      ox[ss] = mx * g.bx;
      const bool wx = mx + 1 == g.Mx;  // carry into y, then z (selects, no branches)
      const bool wy = wx && my + 1 == g.My;
      mx = wx ? 0 : mx + 1;
      my = wy ? 0 : (wx ? my + 1 : my);
      mz = wy ? mz + 1 : mz;
    }
  }
  // RoPE rows of every block of the group: row (ss, axis, local coordinate)
  for (int t = threadIdx.x; t < nrow * P; t += NT) {
    const int row = t / P, pp = t - row * P;
    const int aa = row < g.bz ? 0 : (row < g.bz + g.by ? 1 : 2);
    const int lc = row - (aa == 0 ? 0 : (aa == 1 ? g.bz : g.bz + g.by));
    const int dim = aa == 0 ? g.Z : (aa == 1 ? g.Y : g.X);
    float2 cs[8];
#pragma unroll
    for (int ss = 0; ss < 8; ss++) {
      const int o = aa == 0 ? oz[ss] : (aa == 1 ? oy[ss] : ox[ss]);
      cs[ss] = rope_cs(tab, g, aa, min(o + lc, dim - 1), pp);
    }
#pragma unroll
    for (int ss = 0; ss < 8; ss++) s_cs[(ss * nrow + row) * P + pp] = cs[ss];
  }
  const int rowbase = a == 0 ? 0 : (a == 1 ? g.bz : g.bz + g.by);
  // an absent member reads this 16-byte zero chunk of the geometry buffer
  // instead of a token, so its terms are exact zeros without a select
  const bf16 *zero16 = reinterpret_cast<const bf16 *>(static_cast<const char *>(geom) + kZeroOff);
  // value sums on v_dot2 with weights (1, 0) and (0, 1): one instruction
  // per channel, exactly the fp32 sum of the bf16 values. The weights are
  // kept in registers (the empty asm hides their value): as an inline
  // constant the compiler would encode (1, 0) as the 32-bit constant 1.0,
  // which the instruction reads as the pair (0, 1).
  uint32_t w0 = 0x00003F80u, w1 = 0x3F800000u;  // bf16 pairs (1, 0) and (0, 1)
  asm volatile("" : "+v"(w0), "+v"(w1));
  const bf16x2 e0 = __builtin_bit_cast(bf16x2, w0), e1 = __builtin_bit_cast(bf16x2, w1);
  float ka[8], va[8];
#pragma unroll
  for (int u = 0; u < 8; u++) ka[u] = va[u] = 0.f;
  int cnt = 0;
  const int64_t rowoff = (int64_t)b * g.N;
  for (int r0 = 0; r0 < g.vol; r0 += per) {
    const int nr = min(per, g.vol - r0);
    if (r0 > 0) __syncthreads();  // previous pass done with s_slot, s_lc
    // slots of member rr of every block, and rr's local coordinates
    for (int t = threadIdx.x; t < nr; t += NT) {
      const int rr = r0 + t;
      const int lz = rr / (g.by * g.bx), rem = rr - lz * (g.by * g.bx);
      const int ly = rem / g.bx, lx = rem - ly * g.bx;
      s_lc[t] = lz | (ly << 10) | (lx << 20);
      int j[8];
#pragma unroll
      for (int ss = 0; ss < 8; ss++) {
        const int z = oz[ss] + lz, y = oy[ss] + ly, x = ox[ss] + lx;
        const bool on = m0 + ss < g.M && z < g.Z && y < g.Y && x < g.X;
        j[ss] = slot_get(g, slot, on ? site_of(g, z, y, x) : 0);
        j[ss] = on ? j[ss] : -1;
      }
#pragma unroll
      for (int ss = 0; ss < 8; ss++) s_slot[ss * nr + t] = j[ss];
    }
    __syncthreads();
    for (int q0 = 0; q0 < nr; q0 += kBatch) {
      bf16x8 kr[kBatch], vr[kBatch];
      int jj[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; t++) {
        jj[t] = q0 + t < nr ? s_slot[s * nr + q0 + t] : -1;
        const int64_t off = ((rowoff + max(jj[t], 0)) * g.Hkv + h) * g.D + d0;
        const bool on = jj[t] >= 0;
        kr[t] = *reinterpret_cast<const bf16x8 *>(on ? k + off : zero16);
        vr[t] = *reinterpret_cast<const bf16x8 *>(on ? v + off : zero16);
      }
#pragma unroll
      for (int t = 0; t < kBatch; t++) {
        cnt += jj[t] >= 0 ? 1 : 0;
        const int lcp = s_lc[min(q0 + t, nr - 1)];
        const int lc = (lcp >> (10 * a)) & 1023;
        const float2 *cs = s_cs + ((s * nrow) + rowbase + lc) * P + p0;
#pragma unroll
        for (int u = 0; u < 4; u++) {
          bf16x2 kp, vp;
          kp[0] = kr[t][2 * u];
          kp[1] = kr[t][2 * u + 1];
          vp[0] = vr[t][2 * u];
          vp[1] = vr[t][2 * u + 1];
          if constexpr (CENTRE) {
            ka[2 * u] = __builtin_amdgcn_fdot2_f32_bf16(kp, e0, ka[2 * u], false);
            ka[2 * u + 1] = __builtin_amdgcn_fdot2_f32_bf16(kp, e1, ka[2 * u + 1], false);
          } else {
            // the rotated pair accumulated term by term:
            // (x0 c - x1 s, x0 s + x1 c)
            const float x0 = (float)kp[0], x1 = (float)kp[1];
            const float2 r = cs[u];
            ka[2 * u] = fmaf(-x1, r.y, fmaf(x0, r.x, ka[2 * u]));
            ka[2 * u + 1] = fmaf(x1, r.x, fmaf(x0, r.y, ka[2 * u + 1]));
          }
          va[2 * u] = __builtin_amdgcn_fdot2_f32_bf16(vp, e0, va[2 * u], false);
          va[2 * u + 1] = __builtin_amdgcn_fdot2_f32_bf16(vp, e1, va[2 * u + 1], false);
        }
      }
    }
  }
  // mean = sum / count: one reciprocal per block, then the quotient with
  // one residual correction (exact for a power-of-two count); empty -> 0
  const float fc = (float)cnt;
  const float rc = cnt > 0 ? 1.0f / fc : 0.0f;
  auto mean = [&](float x) {
    const float q = x * rc;
    return fmaf(fmaf(-q, fc, x), rc, q);
  };
  float km[8];
#pragma unroll
  for (int u = 0; u < 8; u++) km[u] = mean(ka[u]);
  if (CENTRE && m < g.M)  // padding slots stay 0 (and have no extent)
    rotate_at_centre<8>(g, m, a, p0, tab,
                        [&](int l, int p) { return s_cs[(s * nrow + rowbase + l) * P + p]; }, km);
  bf16x8 ko;
#pragma unroll
  for (int u = 0; u < 8; u++) {
    ko[u] = (bf16)km[u];
    s_vt[(u * NC + c) * 9 + s] = mean(va[u]);
  }
  {  // m < Mp always: the grid covers Mp / 8 groups
    const int64_t bh = (int64_t)b * g.Hkv + h;
    *reinterpret_cast<bf16x8 *>(ks + ((bh * (Mp / 32) + m / 32) * (g.D / 8) + d0 / 8) * 256 +
                                (m % 32) * 8) = ko;
  }
  __syncthreads();
  // v_sum: one 16-byte chunk per (head, channel) of the group; thread t
  // takes channel 8*(t / 8)... of the row in chunk-major order
  for (int t = threadIdx.x; t < NT; t += NT) {
    const int cc = t >> 3, u = t & 7;          // chunk, channel within it
    const int hh = (cc * 8) / g.D, d = cc * 8 - hh * g.D + u;
    bf16x8 o;
#pragma unroll
    for (int q = 0; q < 8; q++) o[q] = (bf16)s_vt[(u * NC + cc) * 9 + q];
    *reinterpret_cast<bf16x8 *>(vsb + ((((int64_t)b * g.Hkv + hh) * (Mp / 8) + g8) * g.D + d) * 8) = o;
  }
}

namespace {
template <typename T, int CW>
hipError_t run_summarize(const Geo &g, const void *geom, const void *k, const void *v, void *ks,
                         void *vs, hipStream_t s) {
  const int NC = g.Hkv * g.D / CW;
  const int cpt = NC < 64 ? NC : 64;  // chunk lanes per block
  const size_t lds = (size_t)g.Hkv * g.D * 8 * sizeof(float);
  dim3 grid((unsigned)((g.M + 31) / 32 * 4), (unsigned)g.B);
  auto kern = (g.flags & PACK3D_SUMMARY_CENTRE) ? k_summarize<T, CW, true> : k_summarize<T, CW, false>;
  hipLaunchKernelGGL(kern, grid, dim3(8 * cpt), lds, s, g, geom, static_cast<const T *>(k),
                     static_cast<const T *>(v), static_cast<T *>(ks), static_cast<T *>(vs));
  return hipGetLastError();
}
}  // namespace

hipError_t launch_summarize(const Geo &g, int dtype, const void *geom, const void *k,
                            const void *v, void *ks, void *vs, hipStream_t s) {
  // host checks H*D <= 1024, so the transposition buffer stays within 32 KiB
  const bool c8 = g.D % 8 == 0;
  if (dtype == PACK3D_BF16 && c8) {
    const int nrow = g.bz + g.by + g.bx;
    const int per = g.vol < kMaxMembers / 8 ? g.vol : kMaxMembers / 8;
    const size_t lds = (size_t)9 * per * 4 + 8 + (size_t)8 * nrow * g.P * 8 +
                       (size_t)8 * (g.Hkv * g.D / 8) * 9 * 4;
    if (lds <= 48 * 1024 && g.Hkv * g.D <= 512 && g.bz < 1024 && g.by < 1024 && g.bx < 1024) {
      dim3 grid((unsigned)((g.M + 31) / 32 * 4), (unsigned)g.B);
      auto kern = (g.flags & PACK3D_SUMMARY_CENTRE) ? k_summarize_b8<true> : k_summarize_b8<false>;
      hipLaunchKernelGGL(kern, grid, dim3(g.Hkv * g.D), lds, s, g, geom,
                         static_cast<const bf16 *>(k), static_cast<const bf16 *>(v),
                         static_cast<bf16 *>(ks), static_cast<bf16 *>(vs), nrow);
      return hipGetLastError();
    }
  }
  if (dtype == PACK3D_BF16)
    return c8 ? run_summarize<bf16, 8>(g, geom, k, v, ks, vs, s)
              : run_summarize<bf16, 2>(g, geom, k, v, ks, vs, s);
  return c8 ? run_summarize<float, 8>(g, geom, k, v, ks, vs, s)
            : run_summarize<float, 2>(g, geom, k, v, ks, vs, s);
}

}  // namespace pk
