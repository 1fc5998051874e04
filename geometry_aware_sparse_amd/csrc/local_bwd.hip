// Local branch of the backward for bf16 rows of 48 or 96 channels (Geometry
// Matters in Packed 3D Attention: exact 3x3x3 local attention, project page
// Ch. 3, Contract 1; its gradients, paper summary §3.4), laid out like the
// forward's k_local_pair: D/24 lanes per site, each owning 24 consecutive
// channels; dot products by v_dot2_f32_bf16 with the lanes of a site met by
// DPP swaps; sums over neighbours taken two neighbours at a time with one
// v_dot2 per channel (the pair formed by v_perm_b32).
//
//   k_bwd_local_q_pair   per query site: logits as the forward computes them
//                        (rotated, scaled, bf16-rounded q~ against the staged
//                        rotated keys), P in fp32, u_j = <dO, v_j>,
//                        dq = R^T (s sum_j dS_j k~_j + dq~_glob), dG, and
//                        the log-sum-exp and Delta for the key side
//   k_bwd_local_kv_pair  per key site: for every query head of the KV head's
//                        group, the neighbour queries are staged (rotated,
//                        scaled, bf16-rounded exactly as the query side rounds
//                        its own) with dO and the per-site statistics; the
//                        logits are recomputed bit for bit (the same products
//                        summed in the same order), then
//                        dk~ += s dS q~, dv += P (1 - g) dO, and the pooling
//                        and RoPE transposes
//   k_bwd_local_q_tr48   the query side at head dim 48 with dq~ on the matrix
//                        cores
//   k_bwd_local_kv_tr48  the key side at head dim 48 with those two sums on
//                        the matrix cores (LDS transpose loads of the staged
//                        q~ and dO rows, the weights placed as runs of three)
#include "launch.hpp"

namespace pk {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int LPQ>
__device__ __forceinline__ float lane_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf,
                                                          0xf, false));  // quad_perm 1,0,3,2
  if constexpr (LPQ == 4)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xf,
                                                            0xf, false));  // 2,3,0,1
  return x;
}

__device__ __forceinline__ void rotate_t(float &x0, float &x1, float2 cs) {
  float y0 = x0 * cs.x + x1 * cs.y;
  float y1 = -x0 * cs.y + x1 * cs.x;
  x0 = y0;
  x1 = y1;
}

// o[c] += w0 * A[c] + w1 * B[c] for the DH channels of two staged bf16 rows
template <int DH>
__device__ __forceinline__ void pair_accumulate(float *o, float w0, float w1, const bf16 *A,
                                                const bf16 *B) {
  bf16x2 pp;
  pp[0] = (bf16)w0;
  pp[1] = (bf16)w1;
  const uint32_t *a = reinterpret_cast<const uint32_t *>(A);
  const uint32_t *b = reinterpret_cast<const uint32_t *>(B);
#pragma unroll
  for (int j = 0; j < DH / 2; j++) {
    const uint32_t x = a[j], y = b[j];
    const uint32_t lo = __builtin_amdgcn_perm(y, x, 0x05040100u);   // (x.lo, y.lo)
    const uint32_t hi = __builtin_amdgcn_perm(y, x, 0x07060302u);   // (x.hi, y.hi)
    o[2 * j] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2, lo), o[2 * j], false);
    o[2 * j + 1] =
        __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2, hi), o[2 * j + 1], false);
  }
}

// An empty asm that takes the N accumulators as read-write operands: the
// products feeding them are issued before it, so a loop that calls this
// after each step keeps only that step's operands live (without it the
// scheduler hoists every step's LDS reads and byte permutes ahead of the
// accumulation and runs out of registers).
template <int N>
__device__ __forceinline__ void pin(float *a) {
#pragma unroll
  for (int d = 0; d < N; d++) asm volatile("" : "+v"(a[d]));
}

// Halo index of neighbour kk (canonical order: dz outermost, dx innermost)
// counted from the site's (-1, -1, -1) corner, never negative: addresses
// formed from one corner base then differ by constants that fit the LDS
// instructions' unsigned offset field, so they need no register each.
__device__ __forceinline__ int halo_from_corner(int kk, int HY, int HX) {
  return (kk / 9) * HY * HX + ((kk / 3) % 3) * HX + kk % 3;
}
}  // namespace

// Stages the slots of the halo box (-1 off the grid) and the (cos, sin) rows
// of its coordinate range; all loads first, then the LDS writes.
template <int NT, int HZ, int HY, int HX, int P>
__device__ __forceinline__ void stage_box(const Geo &g, const int32_t *slot, const float2 *tab,
                                          int z0, int y0, int x0, int *sSlot, float2 *sCS) {
  constexpr int NH = HZ * HY * HX, NTAB = (HZ + HY + HX) * P;
  constexpr int RT = (NTAB + NT - 1) / NT, RSL = (NH + NT - 1) / NT;
  float2 tv[RT];
  int sv[RSL];
#pragma unroll
  for (int r = 0; r < RT; r++) {
    const int e = min((int)threadIdx.x + r * NT, NTAB - 1);
    const int row = e / P, p = e % P;
    int a, c;
    if (row < HZ) { a = 0; c = z0 - 1 + row; }
    else if (row < HZ + HY) { a = 1; c = y0 - 1 + row - HZ; }
    else { a = 2; c = x0 - 1 + row - HZ - HY; }
    const int dim = a == 0 ? g.Z : (a == 1 ? g.Y : g.X);
    tv[r] = rope_cs(tab, g, a, min(max(c, 0), dim - 1), p);
  }
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
  for (int r = 0; r < RT; r++)
    if ((int)threadIdx.x + r * NT < NTAB) sCS[threadIdx.x + r * NT] = tv[r];
#pragma unroll
  for (int r = 0; r < RSL; r++)
    if ((int)threadIdx.x + r * NT < NH) sSlot[threadIdx.x + r * NT] = sv[r];
}

// ---------------------------------------------------------------------------
template <int D, int TZ, int TY, int TX>
__global__ __launch_bounds__((D / 24) * TZ *TY *TX, D == 48 ? 3 : 2) void k_bwd_local_q_pair(
    Geo g, const void *geom, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const bf16 *__restrict__ gate, const bf16 *__restrict__ dout,
    const bf16 *__restrict__ oglob, const float *__restrict__ dqg, bf16 *dq, bf16 *dgate,
    float *lse_l, float *delta_l, int ntz, int nty, int ntx) {
  constexpr int HZ = TZ + 2, HY = TY + 2, HX = TX + 2, NH = HZ * HY * HX, NQ = TZ * TY * TX;
  constexpr int LPQ = D / 24, NT = LPQ * NQ, DA = D / 3, DH = 24, P = D / 6;
  constexpr int CPS = D / 8, NCK = NH * CPS, RS = (NCK + NT - 1) / NT;
  static_assert(D % 48 == 0 && (LPQ == 2 || LPQ == 4), "head dim 48 or 96");
  // one LDS buffer holds the values for u_j = <dO, v_j>, then the rotated
  // keys for the logits and dq, so that more workgroups fit a CU
  __shared__ __attribute__((aligned(16))) bf16 sK[RS * NT * 8];
  const bf16 *sV = sK;
  __shared__ int sSlot[NH];
  __shared__ float2 sCS[(HZ + HY + HX) * P];

  const BoxWork wk = box_work(xcd_remap(blockIdx.x, gridDim.x), g.H, ntz, nty, ntx);
  const int h = wk.h, b = wk.b;
  const int hk = h / g.G;
  const int z0 = wk.tz * TZ, y0 = wk.ty * TY, x0 = wk.tx * TX;
  const int64_t bN = (int64_t)b * g.N;
  auto cs_at = [&](int a, int rc, int p) {
    const int base = a == 0 ? 0 : (a == 1 ? HZ : HZ + HY);
    return sCS[(base + rc) * P + p];
  };
  stage_box<NT, HZ, HY, HX, P>(g, slot_map(geom, g), rope_table(geom, g), z0, y0, x0, sSlot, sCS);
  __syncthreads();

  const int qn = threadIdx.x / LPQ, hh = threadIdx.x % LPQ;
  const int tz = qn / (TY * TX), ty = (qn / TX) % TY, tx = qn % TX;
  const int qs = ((tz + 1) * HY + (ty + 1)) * HX + (tx + 1);
  const int qc = (tz * HY + ty) * HX + tx;  // the query's (-1, -1, -1) corner
  const int i = sSlot[qs];
  const int wbase = __builtin_amdgcn_readfirstlane(threadIdx.x & ~63);
  // global loads first: raw K chunks, V straight to LDS, this lane's q and dO
  // slices and the gate (O_glob and dq~_glob, needed only at the end, are
  // loaded after the neighbour loop so they hold no registers through it)
  bf16x8 kraw[RS];
#pragma unroll
  for (int r = 0; r < RS; r++) {
    const int e = min((int)threadIdx.x + r * NT, NCK - 1);
    const int hs = e / CPS, ch = e % CPS;
    const int64_t off = ((bN + max(sSlot[hs], 0)) * g.Hkv + hk) * D + ch * 8;
    kraw[r] = *reinterpret_cast<const bf16x8 *>(k + off);
    __builtin_amdgcn_global_load_lds(v + off, (lds_ptr)&sK[(wbase + r * NT) * 8], 16, 0, 0);
  }
  const int64_t row = (bN + max(i, 0)) * g.H + h;
  const int64_t off = row * D + hh * DH;
  bf16x8 qraw[DH / 8], draw[DH / 8];
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) {
    qraw[c8] = *reinterpret_cast<const bf16x8 *>(q + off + 8 * c8);
    draw[c8] = *reinterpret_cast<const bf16x8 *>(dout + off + 8 * c8);
  }
  const float gl = (float)gate[row];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // every lane runs to the end (the barriers below need the whole
  // workgroup); a query site off the grid stores nothing
  const float qscale = g.scale * kLog2e;
  const int rc3[3] = {tz + 1, ty + 1, tx + 1};

  bf16x2 qp[DH / 2], dp[DH / 2];
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) {
    const int d0 = hh * DH + 8 * c8, a = d0 / DA, p0 = (d0 % DA) / 2;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      float x0 = (float)qraw[c8][2 * u], x1 = (float)qraw[c8][2 * u + 1];
      rotate(x0, x1, cs_at(a, rc3[a], p0 + u));
      qp[4 * c8 + u][0] = (bf16)(x0 * qscale);
      qp[4 * c8 + u][1] = (bf16)(x1 * qscale);
      dp[4 * c8 + u][0] = draw[c8][2 * u];
      dp[4 * c8 + u][1] = draw[c8][2 * u + 1];
    }
  }
  // u_j = <dO, v_j>, canonical offset order, from the staged values
  float lg[27], uu[27];
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    const int hs = qc + halo_from_corner(kk, HY, HX);
    const bf16x2 *vr = reinterpret_cast<const bf16x2 *>(sV + hs * D + hh * DH);
    float a1 = 0.f;
#pragma unroll
    for (int j = 0; j < DH / 2; j++) a1 = __builtin_amdgcn_fdot2_f32_bf16(dp[j], vr[j], a1, false);
    uu[kk] = lane_sum<LPQ>(a1);
    // a compiler-only fence per neighbour: the rows of the next ones are not
    // loaded early, which would hold dozens of registers
    asm volatile("" ::: "memory");
  }
  __syncthreads();  // the values are no longer read: the buffer takes the keys
  // rotate the staged keys at their own coordinates, as the forward does
#pragma unroll
  for (int r = 0; r < RS; r++) {
    const int e = (int)threadIdx.x + r * NT;
    const int ec = min(e, NCK - 1);
    const int hs = ec / CPS, ch = ec % CPS;
    const int rc3[3] = {hs / (HY * HX), (hs / HX) % HY, hs % HX};
    const int a = (ch * 8) / DA, p0 = ((ch * 8) % DA) / 2;
    bf16x8 ko;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      float k0 = (float)kraw[r][2 * u], k1 = (float)kraw[r][2 * u + 1];
      rotate(k0, k1, cs_at(a, rc3[a], p0 + u));
      ko[2 * u] = (bf16)k0;
      ko[2 * u + 1] = (bf16)k1;
    }
    *reinterpret_cast<bf16x8 *>(&sK[e * 8]) = ko;
  }
  __syncthreads();
  // logits (log2 units), canonical offset order
  float mx = -INFINITY;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    const int hs = qc + halo_from_corner(kk, HY, HX);
    const bf16x2 *kr = reinterpret_cast<const bf16x2 *>(sK + hs * D + hh * DH);
    float a0 = 0.f;
#pragma unroll
    for (int j = 0; j < DH / 2; j++) a0 = __builtin_amdgcn_fdot2_f32_bf16(qp[j], kr[j], a0, false);
    a0 = lane_sum<LPQ>(a0);
    lg[kk] = sSlot[hs] >= 0 ? a0 : -INFINITY;
    mx = fmaxf(mx, lg[kk]);
    asm volatile("" ::: "memory");
  }
  float den = 0.f;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    lg[kk] = __builtin_amdgcn_exp2f(lg[kk] - mx);  // 0 for an invalid neighbour
    den += lg[kk];
  }
  const float inv = 1.0f / den;
  asm volatile("" ::: "memory");  // the next phase re-reads its rows from LDS
  float dol = 0.f;  // <dO, O_loc>
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    lg[kk] *= inv;
    dol += lg[kk] * uu[kk];
  }
  const float gg = 1.0f / (1.0f + expf(-gl)), omg = 1.0f - gg;
  const float delta = omg * dol;
  // dq~ = sum_j dS_j k~_j, two neighbours per step (the last step's second
  // member has weight 0)
  float acc[DH];
#pragma unroll
  for (int d = 0; d < DH; d++) acc[d] = 0.f;
#pragma unroll
  for (int kp = 0; kp < 14; kp++) {
    const int k0 = 2 * kp, k1 = kp < 13 ? 2 * kp + 1 : 2 * kp;
    const float w0 = lg[k0] * (omg * uu[k0] - delta);
    const float w1 = kp < 13 ? lg[k1] * (omg * uu[k1] - delta) : 0.f;
    pair_accumulate<DH>(acc, w0, w1, sK + (qc + halo_from_corner(k0, HY, HX)) * D + hh * DH,
                        sK + (qc + halo_from_corner(k1, HY, HX)) * D + hh * DH);
    pin<DH>(acc);
    asm volatile("" ::: "memory");
  }
  if (i < 0) return;
  // dq = R^T (s dq~_loc + dq~_glob); dG = g (1 - g) (<dO, O_glob> - <dO, O_loc>)
  bf16x8 oraw[DH / 8];
  f32x4 gq[DH / 4];
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) oraw[c8] = *reinterpret_cast<const bf16x8 *>(oglob + off + 8 * c8);
#pragma unroll
  for (int c4 = 0; c4 < DH / 4; c4++) gq[c4] = *reinterpret_cast<const f32x4 *>(dqg + off + 4 * c4);
  float dgo = 0.f;
  bf16x8 outv[DH / 8];
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) {
    const int d0 = hh * DH + 8 * c8, a = d0 / DA, p0 = (d0 % DA) / 2;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int c = 8 * c8 + 2 * u;
      float x0 = g.scale * acc[c] + gq[c / 4][c % 4];
      float x1 = g.scale * acc[c + 1] + gq[(c + 1) / 4][(c + 1) % 4];
      rotate_t(x0, x1, cs_at(a, rc3[a], p0 + u));
      outv[c8][2 * u] = (bf16)x0;
      outv[c8][2 * u + 1] = (bf16)x1;
    }
#pragma unroll
    for (int e = 0; e < 8; e++) dgo += (float)draw[c8][e] * (float)oraw[c8][e];
  }
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) *reinterpret_cast<bf16x8 *>(dq + off + 8 * c8) = outv[c8];
  dgo = lane_sum<LPQ>(dgo);
  if (hh == 0) {
    dgate[row] = (bf16)(gg * omg * (dgo - dol));
    lse_l[row] = mx + __log2f(den);
    delta_l[row] = delta;
  }
}

// ---------------------------------------------------------------------------
// The query side at head dim 48 with dq~ = sum_j dS_j k~_j on the matrix
// cores, as k_bwd_local_kv_tr48 sums over neighbour queries; the logits,
// u_j, the softmax, dG and the statistics are those of k_bwd_local_q_pair.
__global__ __launch_bounds__(256, 3) void k_bwd_local_q_tr48(
    Geo g, const void *geom, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const bf16 *__restrict__ gate, const bf16 *__restrict__ dout,
    const bf16 *__restrict__ oglob, const float *__restrict__ dqg, bf16 *dq, bf16 *dgate,
    float *lse_l, float *delta_l, int ntz, int nty, int ntx) {
  constexpr int D = 48, TZ = 4, TY = 4, TX = 8;
  constexpr int HZ = TZ + 2, HY = TY + 2, HX = TX + 2, NPL = HY * HX, NH = HZ * NPL, NQ = TZ * TY * TX;
  constexpr int LPQ = 2, NT = LPQ * NQ, DA = D / 3, DH = 24, P = D / 6;
  constexpr int CPS = D / 8, NCK = NH * CPS, RS = (NCK + NT - 1) / NT;
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s *lds_v4s;
  // one LDS buffer holds the values for u_j = <dO, v_j>, then the rotated
  // keys for the logits and dq, so that more workgroups fit a CU
  __shared__ __attribute__((aligned(16))) bf16 sK[RS * NT * 8];
  const bf16 *sV = sK;
  __shared__ int sSlot[NH];
  __shared__ float2 sCS[(HZ + HY + HX) * P];
  // the furthest operand read: padding site 63 of the last plane, channel 63
  static_assert(((HZ - 1) * NPL + 64) * D + (64 - D) <= RS * NT * 8,
                "padding sites and channels stay in the buffer");

  const BoxWork wk = box_work(xcd_remap(blockIdx.x, gridDim.x), g.H, ntz, nty, ntx);
  const int h = wk.h, b = wk.b;
  const int hk = h / g.G;
  const int z0 = wk.tz * TZ, y0 = wk.ty * TY, x0 = wk.tx * TX;
  const int64_t bN = (int64_t)b * g.N;
  auto cs_at = [&](int a, int rc, int p) {
    const int base = a == 0 ? 0 : (a == 1 ? HZ : HZ + HY);
    return sCS[(base + rc) * P + p];
  };
  stage_box<NT, HZ, HY, HX, P>(g, slot_map(geom, g), rope_table(geom, g), z0, y0, x0, sSlot, sCS);
  __syncthreads();

  const int qn = threadIdx.x / LPQ, hh = threadIdx.x % LPQ;
  const int tz = qn / (TY * TX), ty = (qn / TX) % TY, tx = qn % TX;
  const int qs = ((tz + 1) * HY + (ty + 1)) * HX + (tx + 1);
  const int qc = (tz * HY + ty) * HX + tx;  // the query's (-1, -1, -1) corner
  const int i = sSlot[qs];
  const int wbase = __builtin_amdgcn_readfirstlane(threadIdx.x & ~63);
  // global loads first: raw K chunks, V straight to LDS, this lane's q and dO
  // slices and the gate (O_glob and dq~_glob, needed only at the end, are
  // loaded after the neighbour loop so they hold no registers through it)
  bf16x8 kraw[RS];
#pragma unroll
  for (int r = 0; r < RS; r++) {
    const int e = min((int)threadIdx.x + r * NT, NCK - 1);
    const int hs = e / CPS, ch = e % CPS;
    const int64_t off = ((bN + max(sSlot[hs], 0)) * g.Hkv + hk) * D + ch * 8;
    kraw[r] = *reinterpret_cast<const bf16x8 *>(k + off);
    __builtin_amdgcn_global_load_lds(v + off, (lds_ptr)&sK[(wbase + r * NT) * 8], 16, 0, 0);
  }
  const int64_t row = (bN + max(i, 0)) * g.H + h;
  const int64_t off = row * D + hh * DH;
  bf16x8 qraw[DH / 8], draw[DH / 8];
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) {
    qraw[c8] = *reinterpret_cast<const bf16x8 *>(q + off + 8 * c8);
    draw[c8] = *reinterpret_cast<const bf16x8 *>(dout + off + 8 * c8);
  }
  const float gl = (float)gate[row];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // every lane runs to the end (the barriers below need the whole
  // workgroup); a query site off the grid stores nothing
  const float qscale = g.scale * kLog2e;
  const int rc3[3] = {tz + 1, ty + 1, tx + 1};

  bf16x2 qp[DH / 2], dp[DH / 2];
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) {
    const int d0 = hh * DH + 8 * c8, a = d0 / DA, p0 = (d0 % DA) / 2;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      float x0 = (float)qraw[c8][2 * u], x1 = (float)qraw[c8][2 * u + 1];
      rotate(x0, x1, cs_at(a, rc3[a], p0 + u));
      qp[4 * c8 + u][0] = (bf16)(x0 * qscale);
      qp[4 * c8 + u][1] = (bf16)(x1 * qscale);
      dp[4 * c8 + u][0] = draw[c8][2 * u];
      dp[4 * c8 + u][1] = draw[c8][2 * u + 1];
    }
  }
  // u_j = <dO, v_j>, canonical offset order, from the staged values
  float lg[27], uu[27];
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    const int hs = qc + halo_from_corner(kk, HY, HX);
    const bf16x2 *vr = reinterpret_cast<const bf16x2 *>(sV + hs * D + hh * DH);
    float a1 = 0.f;
#pragma unroll
    for (int j = 0; j < DH / 2; j++) a1 = __builtin_amdgcn_fdot2_f32_bf16(dp[j], vr[j], a1, false);
    uu[kk] = lane_sum<LPQ>(a1);
    // a compiler-only fence per neighbour: the rows of the next ones are not
    // loaded early, which would hold dozens of registers
    asm volatile("" ::: "memory");
  }
  __syncthreads();  // the values are no longer read: the buffer takes the keys
  // rotate the staged keys at their own coordinates, as the forward does
#pragma unroll
  for (int r = 0; r < RS; r++) {
    const int e = (int)threadIdx.x + r * NT;
    const int ec = min(e, NCK - 1);
    const int hs = ec / CPS, ch = ec % CPS;
    const int rc3[3] = {hs / (HY * HX), (hs / HX) % HY, hs % HX};
    const int a = (ch * 8) / DA, p0 = ((ch * 8) % DA) / 2;
    bf16x8 ko;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      float k0 = (float)kraw[r][2 * u], k1 = (float)kraw[r][2 * u + 1];
      rotate(k0, k1, cs_at(a, rc3[a], p0 + u));
      ko[2 * u] = (bf16)k0;
      ko[2 * u + 1] = (bf16)k1;
    }
    *reinterpret_cast<bf16x8 *>(&sK[e * 8]) = ko;
  }
  __syncthreads();
  // logits (log2 units), canonical offset order
  float mx = -INFINITY;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    const int hs = qc + halo_from_corner(kk, HY, HX);
    const bf16x2 *kr = reinterpret_cast<const bf16x2 *>(sK + hs * D + hh * DH);
    float a0 = 0.f;
#pragma unroll
    for (int j = 0; j < DH / 2; j++) a0 = __builtin_amdgcn_fdot2_f32_bf16(qp[j], kr[j], a0, false);
    a0 = lane_sum<LPQ>(a0);
    lg[kk] = sSlot[hs] >= 0 ? a0 : -INFINITY;
    mx = fmaxf(mx, lg[kk]);
    asm volatile("" ::: "memory");
  }
  float den = 0.f;
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    lg[kk] = __builtin_amdgcn_exp2f(lg[kk] - mx);  // 0 for an invalid neighbour
    den += lg[kk];
  }
  const float inv = 1.0f / den;
  asm volatile("" ::: "memory");  // the next phase re-reads its rows from LDS
  float dol = 0.f;  // <dO, O_loc>
#pragma unroll
  for (int kk = 0; kk < 27; kk++) {
    lg[kk] *= inv;
    dol += lg[kk] * uu[kk];
  }
  const float gg = 1.0f / (1.0f + expf(-gl)), omg = 1.0f - gg;
  const float delta = omg * dol;
  // dq~ = sum_j dS_j k~_j on the matrix cores: the bf16 weights dS as
  // triples (dx = -1, 0, +1) of each (dz, dy), packed as the words (w-, w0)
  // and (w+, 0), moved to the product layout (lanes n, n + 32 for query n),
  // then dq~^T (two 32-row tiles of channels x 32 queries) += K~^T * dS^T
  // over the 3 planes x 4 blocks of 16 sites a plane of queries can see
  uint32_t tD[9][2];
#pragma unroll
  for (int r9 = 0; r9 < 9; r9++) {
    float w3[3];
#pragma unroll
    for (int dx = 0; dx < 3; dx++) {
      const int kk = 3 * r9 + dx;
      w3[dx] = lg[kk] * (omg * uu[kk] - delta);  // 0 for an invalid neighbour
    }
    bf16x2 t0, t1;
    t0[0] = (bf16)w3[0];
    t0[1] = (bf16)w3[1];
    t1[0] = (bf16)w3[2];
    t1[1] = (bf16)0.0f;
    tD[r9][0] = __builtin_bit_cast(uint32_t, t0);
    tD[r9][1] = __builtin_bit_cast(uint32_t, t1);
  }
  const int lane = threadIdx.x & 63;
  const int hi = lane >> 5, ql = lane & 31;
  const int pty = ql >> 3, ptx = ql & 7;
#pragma unroll
  for (int r9 = 0; r9 < 9; r9++)
#pragma unroll
    for (int w = 0; w < 2; w++) tD[r9][w] = (uint32_t)__shfl((int)tD[r9][w], 2 * ql);
  f32x16 acc2[2];
#pragma unroll
  for (int t2 = 0; t2 < 2; t2++)
#pragma unroll
    for (int e = 0; e < 16; e++) acc2[t2][e] = 0.f;
  {
    const int grp = (lane >> 4) & 1, rq = lane & 3, re = (lane >> 2) & 3;
    const int abase = (tz * NPL + re) * D + 16 * grp + 4 * rq;  // elements
#pragma unroll
    for (int kb4 = 0; kb4 < 4; kb4++) {
      // this lane's window: sites kappa0 = 16*kb4 + 8*hi .. +7 of a plane
      // (kappa = y*10 + x); at most one run of the query's neighbour rows
      // meets it, at slot offset o in [-2, 7]
      const int k0 = 16 * kb4 + 8 * hi;
      const int sm = pty * 10 + ptx;
      const int rel = k0 - sm + 7;
      const int di = rel >= 0 ? rel / 10 : -1;
      const bool ok = di >= 0 && di <= 2;
      const int o = sm + 10 * di - k0;
      const int m = ok ? (o >> 1) : -8;
      const bool odd = (o & 1) != 0;
      const uint32_t s0 = odd ? 0x01000C0Cu : 0x03020100u, s1 = odd ? 0x05040302u : 0x07060504u;
      uint32_t sel[4];
#pragma unroll
      for (int jd = 0; jd < 4; jd++) sel[jd] = jd == m ? s0 : (jd == m + 1 ? s1 : 0x0C0C0C0Cu);
#pragma unroll
      for (int dzi = 0; dzi < 3; dzi++) {
        const uint32_t x0 = di == 0 ? tD[3 * dzi][0] : (di == 1 ? tD[3 * dzi + 1][0] : tD[3 * dzi + 2][0]);
        const uint32_t x1 = di == 0 ? tD[3 * dzi][1] : (di == 1 ? tD[3 * dzi + 1][1] : tD[3 * dzi + 2][1]);
        uint32_t bw[4];
#pragma unroll
        for (int jd = 0; jd < 4; jd++) bw[jd] = __builtin_amdgcn_perm(x1, x0, sel[jd]);
        bf16x8 bop;
        __builtin_memcpy(&bop, bw, 16);
#pragma unroll
        for (int t2 = 0; t2 < 2; t2++) {
          const int ad = abase + (dzi * NPL + k0) * D + 32 * t2;
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(sK + ad));
          const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(sK + ad + 4 * D));
          bf16x8 aop;
          __builtin_memcpy(&aop, &lo, 8);
          __builtin_memcpy(reinterpret_cast<char *>(&aop) + 8, &hi4, 8);
          acc2[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, acc2[t2], 0, 0, 0);
        }
      }
    }
  }
  // Lane (n, hi) holds channels 8*jj + 4*hi .. +3 of query n (tile jj / 4,
  // registers 4*(jj % 4) ..); the halves trade pieces (v_permlane32_swap) so
  // that each lane holds channels 16*mm + 8*hi .. +7, mm = 0, 1, 2.
  float od[3][8];
#pragma unroll
  for (int mm = 0; mm < 3; mm++)
#pragma unroll
    for (int u = 0; u < 4; u++) {
      // elements copied out first: a bit cast applied straight to a vector
      // element subscript compiles to a cast of element 0
      const float e0 = acc2[(2 * mm) / 4][4 * ((2 * mm) % 4) + u];
      const float e1 = acc2[(2 * mm + 1) / 4][4 * ((2 * mm + 1) % 4) + u];
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, e0),
                                                       __builtin_bit_cast(uint32_t, e1), false, false);
      od[mm][u] = __builtin_bit_cast(float, (uint32_t)sw[0]);
      od[mm][4 + u] = __builtin_bit_cast(float, (uint32_t)sw[1]);
    }
  // dq = R^T (s dq~_loc + dq~_glob) for query n = ql of plane tz
  {
    const int pi = sSlot[((tz + 1) * HY + (pty + 1)) * HX + (ptx + 1)];
    if (pi >= 0) {
      const int prc3[3] = {tz + 1, pty + 1, ptx + 1};
      const int64_t poff = ((bN + pi) * g.H + h) * D;
#pragma unroll
      for (int mm = 0; mm < 3; mm++) {
        const int d0 = 16 * mm + 8 * hi;  // axis chunk mm, its planes 4*hi ..
        const f32x4 g0 = *reinterpret_cast<const f32x4 *>(dqg + poff + d0);
        const f32x4 g1 = *reinterpret_cast<const f32x4 *>(dqg + poff + d0 + 4);
        const float gf[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        bf16x8 ov;
#pragma unroll
        for (int u = 0; u < 4; u++) {
          float x0 = g.scale * od[mm][2 * u] + gf[2 * u];
          float x1 = g.scale * od[mm][2 * u + 1] + gf[2 * u + 1];
          rotate_t(x0, x1, cs_at(mm, prc3[mm], 4 * hi + u));
          ov[2 * u] = (bf16)x0;
          ov[2 * u + 1] = (bf16)x1;
        }
        *reinterpret_cast<bf16x8 *>(dq + poff + d0) = ov;
      }
    }
  }
  if (i < 0) return;
  // dG = g (1 - g) (<dO, O_glob> - <dO, O_loc>)
  bf16x8 oraw[DH / 8];
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) oraw[c8] = *reinterpret_cast<const bf16x8 *>(oglob + off + 8 * c8);
  float dgo = 0.f;
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++)
#pragma unroll
    for (int e = 0; e < 8; e++) dgo += (float)draw[c8][e] * (float)oraw[c8][e];
  dgo = lane_sum<LPQ>(dgo);
  if (hh == 0) {
    dgate[row] = (bf16)(gg * omg * (dgo - dol));
    lse_l[row] = mx + __log2f(den);
    delta_l[row] = delta;
  }
}

// ---------------------------------------------------------------------------
template <int D, int TZ, int TY, int TX, bool CENTRE>
__global__ __launch_bounds__((D / 24) * TZ *TY *TX, 2) void k_bwd_local_kv_pair(
    Geo g, const void *geom, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const bf16 *__restrict__ gate, const bf16 *__restrict__ dout,
    const float *__restrict__ lse_l, const float *__restrict__ delta_l,
    const float *__restrict__ dks, const float *__restrict__ dvs, bf16 *dk, bf16 *dv, int ntz,
    int nty, int ntx) {
  constexpr int HZ = TZ + 2, HY = TY + 2, HX = TX + 2, NH = HZ * HY * HX, NQ = TZ * TY * TX;
  constexpr int LPQ = D / 24, NT = LPQ * NQ, DA = D / 3, DH = 24, P = D / 6;
  constexpr int CPS = D / 8, NCK = NH * CPS, RS = (NCK + NT - 1) / NT, RSL = (NH + NT - 1) / NT;
  static_assert(D % 48 == 0 && (LPQ == 2 || LPQ == 4), "head dim 48 or 96");
  __shared__ __attribute__((aligned(16))) bf16 sQ[RS * NT * 8];
  __shared__ __attribute__((aligned(16))) bf16 sO[RS * NT * 8];
  __shared__ int sSlot[NH];
  __shared__ float2 sCS[(HZ + HY + HX) * P];
  __shared__ float sOmg[NH], sL[NH], sDl[NH];

  const BoxWork wk = box_work(xcd_remap(blockIdx.x, gridDim.x), g.Hkv, ntz, nty, ntx);
  const int hk = wk.h, b = wk.b;
  const int z0 = wk.tz * TZ, y0 = wk.ty * TY, x0 = wk.tx * TX;
  const int64_t bN = (int64_t)b * g.N;
  const float2 *tab = rope_table(geom, g);
  auto cs_at = [&](int a, int rc, int p) {
    const int base = a == 0 ? 0 : (a == 1 ? HZ : HZ + HY);
    return sCS[(base + rc) * P + p];
  };
  stage_box<NT, HZ, HY, HX, P>(g, slot_map(geom, g), tab, z0, y0, x0, sSlot, sCS);
  __syncthreads();

  const int kn = threadIdx.x / LPQ, hh = threadIdx.x % LPQ;
  const int tz = kn / (TY * TX), ty = (kn / TX) % TY, tx = kn % TX;
  const int ks_ = ((tz + 1) * HY + (ty + 1)) * HX + (tx + 1);
  const int j = sSlot[ks_];
  const int rc3[3] = {tz + 1, ty + 1, tx + 1};
  const int wbase = __builtin_amdgcn_readfirstlane(threadIdx.x & ~63);
  const float qscale = g.scale * kLog2e;
  // this key's rotated bf16 slice (as the query side staged it) and values
  const int64_t jrow = (bN + max(j, 0)) * g.Hkv + hk;
  const int64_t joff = jrow * D + hh * DH;
  bf16x2 kp[DH / 2], vp[DH / 2];
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) {
    const bf16x8 kr = *reinterpret_cast<const bf16x8 *>(k + joff + 8 * c8);
    const bf16x8 vr = *reinterpret_cast<const bf16x8 *>(v + joff + 8 * c8);
    const int d0 = hh * DH + 8 * c8, a = d0 / DA, p0 = (d0 % DA) / 2;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      float k0 = (float)kr[2 * u], k1 = (float)kr[2 * u + 1];
      rotate(k0, k1, cs_at(a, rc3[a], p0 + u));
      kp[4 * c8 + u][0] = (bf16)k0;
      kp[4 * c8 + u][1] = (bf16)k1;
      vp[4 * c8 + u][0] = vr[2 * u];
      vp[4 * c8 + u][1] = vr[2 * u + 1];
    }
  }
  float adk[DH], adv[DH];
#pragma unroll
  for (int d = 0; d < DH; d++) adk[d] = adv[d] = 0.f;

  for (int h = hk * g.G; h < (hk + 1) * g.G; h++) {
    __syncthreads();  // the previous head's stage is no longer read
    // all loads first: raw q chunks, dO straight to LDS, per-site statistics
    bf16x8 qraw[RS];
#pragma unroll
    for (int r = 0; r < RS; r++) {
      const int e = min((int)threadIdx.x + r * NT, NCK - 1);
      const int hs = e / CPS, ch = e % CPS;
      const int64_t off = ((bN + max(sSlot[hs], 0)) * g.H + h) * D + ch * 8;
      qraw[r] = *reinterpret_cast<const bf16x8 *>(q + off);
      __builtin_amdgcn_global_load_lds(dout + off, (lds_ptr)&sO[(wbase + r * NT) * 8], 16, 0, 0);
    }
    float st_g[RSL], st_l[RSL], st_d[RSL];
#pragma unroll
    for (int r = 0; r < RSL; r++) {
      const int hs = min((int)threadIdx.x + r * NT, NH - 1);
      const int64_t srow = (bN + max(sSlot[hs], 0)) * g.H + h;
      st_g[r] = (float)gate[srow];
      st_l[r] = lse_l[srow];
      st_d[r] = delta_l[srow];
    }
#pragma unroll
    for (int r = 0; r < RS; r++) {
      const int e = (int)threadIdx.x + r * NT;
      const int ec = min(e, NCK - 1);
      const int hs = ec / CPS, ch = ec % CPS;
      const int qc3[3] = {hs / (HY * HX), (hs / HX) % HY, hs % HX};
      const int a = (ch * 8) / DA, p0 = ((ch * 8) % DA) / 2;
      bf16x8 qo;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        float x0 = (float)qraw[r][2 * u], x1 = (float)qraw[r][2 * u + 1];
        rotate(x0, x1, cs_at(a, qc3[a], p0 + u));
        qo[2 * u] = (bf16)(x0 * qscale);
        qo[2 * u + 1] = (bf16)(x1 * qscale);
      }
      *reinterpret_cast<bf16x8 *>(&sQ[e * 8]) = qo;
    }
#pragma unroll
    for (int r = 0; r < RSL; r++) {
      const int hs = (int)threadIdx.x + r * NT;
      if (hs < NH) {
        sOmg[hs] = 1.0f - 1.0f / (1.0f + expf(-st_g[r]));
        sL[hs] = st_l[r];
        sDl[hs] = st_d[r];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j < 0) continue;
    // the key's corner index, opaque to the compiler within this head: the
    // 27 neighbour addresses derived from it are formed here rather than
    // hoisted out of the head loop, where they would hold ~100 registers
    int ksh = ((tz * HY) + ty) * HX + tx;  // the key's (-1, -1, -1) corner
    asm volatile("" : "+v"(ksh));
    // logits (the query side's, bit for bit) and u_ij = <dO_i, v_j>
    float pw[27], dsw[27];
#pragma unroll
    for (int kk = 0; kk < 27; kk++) {
      const int hs = ksh + halo_from_corner(kk, HY, HX);
      const bf16x2 *qr = reinterpret_cast<const bf16x2 *>(sQ + hs * D + hh * DH);
      const bf16x2 *orr = reinterpret_cast<const bf16x2 *>(sO + hs * D + hh * DH);
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int jj = 0; jj < DH / 2; jj++) {
        a0 = __builtin_amdgcn_fdot2_f32_bf16(qr[jj], kp[jj], a0, false);
        a1 = __builtin_amdgcn_fdot2_f32_bf16(orr[jj], vp[jj], a1, false);
      }
      a0 = lane_sum<LPQ>(a0);
      a1 = lane_sum<LPQ>(a1);
      const bool valid = sSlot[hs] >= 0;
      const float pr = valid ? __builtin_amdgcn_exp2f(a0 - sL[hs]) : 0.f;
      pw[kk] = pr * sOmg[hs];
      dsw[kk] = pr * (sOmg[hs] * a1 - sDl[hs]);
      pin<1>(&pw[kk]);
      pin<1>(&dsw[kk]);
      asm volatile("" ::: "memory");  // as on the query side
    }
    asm volatile("" ::: "memory");  // the next phase re-reads its rows from LDS
    // dk~ over the staged queries, then dv over the staged dO: one row pair
    // in flight at a time
#pragma unroll
    for (int kp2 = 0; kp2 < 14; kp2++) {
      const int k0 = 2 * kp2, k1 = kp2 < 13 ? 2 * kp2 + 1 : 2 * kp2;
      const int hs0 = ksh + halo_from_corner(k0, HY, HX), hs1 = ksh + halo_from_corner(k1, HY, HX);
      const float c1 = kp2 < 13 ? 1.f : 0.f;
      pair_accumulate<DH>(adk, dsw[k0], c1 * dsw[k1], sQ + hs0 * D + hh * DH, sQ + hs1 * D + hh * DH);
      pin<DH>(adk);
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int kp2 = 0; kp2 < 14; kp2++) {
      const int k0 = 2 * kp2, k1 = kp2 < 13 ? 2 * kp2 + 1 : 2 * kp2;
      const int hs0 = ksh + halo_from_corner(k0, HY, HX), hs1 = ksh + halo_from_corner(k1, HY, HX);
      const float c1 = kp2 < 13 ? 1.f : 0.f;
      pair_accumulate<DH>(adv, pw[k0], c1 * pw[k1], sO + hs0 * D + hh * DH, sO + hs1 * D + hh * DH);
      pin<DH>(adv);
      asm volatile("" ::: "memory");
    }
  }
  if (j < 0) return;
  // pooling transpose, then dk = R(c_j)^T dk~ (centre variant: its block part
  // goes through R(centre)^T instead)
  const int c3[3] = {z0 + tz, y0 + ty, x0 + tx};
  const int m = block_of(g, c3[0], c3[1], c3[2]);
  const int mz = m / (g.My * g.Mx), my = (m / g.Mx) % g.My, mx = m % g.Mx;
  const int nm = min(g.bz, g.Z - mz * g.bz) * min(g.by, g.Y - my * g.by) * min(g.bx, g.X - mx * g.bx);
  const float inv_n = 1.0f / (float)nm;
  const float *gk = dks + ((((int64_t)b * g.Hkv + hk) * g.M + m) * D + hh * DH);
  const float *gv = dvs + ((((int64_t)b * g.Hkv + hk) * g.M + m) * D + hh * DH);
  bf16x8 okv[DH / 8], ovv[DH / 8];
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) {
    const int d0 = hh * DH + 8 * c8, a = d0 / DA, p0 = (d0 % DA) / 2;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int c = 8 * c8 + 2 * u;
      float x0 = kLn2 * adk[c], x1 = kLn2 * adk[c + 1];  // s / (s log2 e)
      if (!CENTRE) {
        x0 += gk[c] * inv_n;
        x1 += gk[c + 1] * inv_n;
      }
      rotate_t(x0, x1, cs_at(a, rc3[a], p0 + u));
      if (CENTRE) {
        const int mzz = m / (g.My * g.Mx), myy = (m / g.Mx) % g.My, mxx = m % g.Mx;
        const int o = a == 0 ? mzz * g.bz : (a == 1 ? myy * g.by : mxx * g.bx);
        const int ext = min(a == 0 ? g.bz : (a == 1 ? g.by : g.bx),
                            (a == 0 ? g.Z : (a == 1 ? g.Y : g.X)) - o);
        float2 t = rope_cs(tab, g, a, o + (ext - 1) / 2, p0 + u);
        if ((ext & 1) == 0) {
          const float2 hf = rope_half(tab, g, p0 + u);
          t = make_float2(t.x * hf.x - t.y * hf.y, t.y * hf.x + t.x * hf.y);
        }
        float y0 = gk[c] * inv_n, y1 = gk[c + 1] * inv_n;
        rotate_t(y0, y1, t);
        x0 += y0;
        x1 += y1;
      }
      okv[c8][2 * u] = (bf16)x0;
      okv[c8][2 * u + 1] = (bf16)x1;
      ovv[c8][2 * u] = (bf16)(adv[c] + gv[c] * inv_n);
      ovv[c8][2 * u + 1] = (bf16)(adv[c + 1] + gv[c + 1] * inv_n);
    }
  }
#pragma unroll
  for (int c8 = 0; c8 < DH / 8; c8++) {
    *reinterpret_cast<bf16x8 *>(dk + joff + 8 * c8) = okv[c8];
    *reinterpret_cast<bf16x8 *>(dv + joff + 8 * c8) = ovv[c8];
  }
}

// ---------------------------------------------------------------------------
// The key side at head dim 48 with its two weighted sums over neighbour
// queries on the matrix cores, as the forward's local kernel sums values.
// The logits, u_ij and the weights are formed exactly as in
// k_bwd_local_kv_pair (lanes 2n, 2n + 1 serve key n, one channel half each);
// then, per wave (the keys of one z-plane of the 4 x 4 x 8 box),
//   dk~^T (two 32-row tiles of channels x 32 keys) += Q~^T * dS^T,
//   dv^T                                           += dO^T * (P (1 - g))^T
// with v_mfma_f32_32x32x16_bf16 over the 3 planes x 4 blocks of 16 sites a
// plane of keys can see. The A operands come from the staged row-major q~
// and dO rows through the LDS transpose load; the B operands hold each key's
// bf16 weights for 8 sites, placed as one run of three (dx = -1, 0, +1) by
// byte permutes. The weights are rounded to bf16 as the vector form rounds
// them; each sum's order is fixed by the key's position in its box.
template <bool CENTRE>
__global__ __launch_bounds__(256, 2) void k_bwd_local_kv_tr48(
    Geo g, const void *geom, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const bf16 *__restrict__ gate, const bf16 *__restrict__ dout,
    const float *__restrict__ lse_l, const float *__restrict__ delta_l,
    const float *__restrict__ dks, const float *__restrict__ dvs, bf16 *dk, bf16 *dv, int ntz,
    int nty, int ntx) {
  constexpr int D = 48, TZ = 4, TY = 4, TX = 8;
  constexpr int HZ = TZ + 2, HY = TY + 2, HX = TX + 2, NPL = HY * HX, NH = HZ * NPL;
  constexpr int LPQ = 2, NT = 256, DA = D / 3, DH = 24, P = D / 6;
  constexpr int CPS = D / 8, NCK = NH * CPS, RS = (NCK + NT - 1) / NT, RSL = (NH + NT - 1) / NT;
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s *lds_v4s;
  __shared__ __attribute__((aligned(16))) bf16 sQ[RS * NT * 8];
  __shared__ __attribute__((aligned(16))) bf16 sO[RS * NT * 8];
  __shared__ int sSlot[NH];
  __shared__ float2 sCS[(HZ + HY + HX) * P];
  __shared__ float sOmg[NH], sL[NH], sDl[NH];
  // the furthest operand read: padding site 63 of the last plane, channel 63
  static_assert(((HZ - 1) * NPL + 64) * D + (64 - D) <= RS * NT * 8,
                "padding sites and channels stay in the buffers");

  const BoxWork wk = box_work(xcd_remap(blockIdx.x, gridDim.x), g.Hkv, ntz, nty, ntx);
  const int hk = wk.h, b = wk.b;
  const int z0 = wk.tz * TZ, y0 = wk.ty * TY, x0 = wk.tx * TX;
  const int64_t bN = (int64_t)b * g.N;
  const float2 *tab = rope_table(geom, g);
  auto cs_at = [&](int a, int rc, int p) {
    const int base = a == 0 ? 0 : (a == 1 ? HZ : HZ + HY);
    return sCS[(base + rc) * P + p];
  };
  stage_box<NT, HZ, HY, HX, P>(g, slot_map(geom, g), tab, z0, y0, x0, sSlot, sCS);
  __syncthreads();

  // logits layout: lanes 2n, 2n + 1 serve key n (channel halves hh)
  const int lane = threadIdx.x & 63;
  const int kn = threadIdx.x / LPQ, hh = threadIdx.x % LPQ;
  const int tz = kn / (TY * TX), ty = (kn / TX) % TY, tx = kn % TX;
  const int ks_ = ((tz + 1) * HY + (ty + 1)) * HX + (tx + 1);
  const int j = sSlot[ks_];
  const int rc3[3] = {tz + 1, ty + 1, tx + 1};
  const int wbase = __builtin_amdgcn_readfirstlane(threadIdx.x & ~63);
  const float qscale = g.scale * kLog2e;
  // this key's rotated bf16 slice (as the query side staged it) and values
  bf16x2 kp[DH / 2], vp[DH / 2];
  {
    const int64_t joff = ((bN + max(j, 0)) * g.Hkv + hk) * D + hh * DH;
#pragma unroll
    for (int c8 = 0; c8 < DH / 8; c8++) {
      const bf16x8 kr = *reinterpret_cast<const bf16x8 *>(k + joff + 8 * c8);
      const bf16x8 vr = *reinterpret_cast<const bf16x8 *>(v + joff + 8 * c8);
      const int d0 = hh * DH + 8 * c8, a = d0 / DA, p0 = (d0 % DA) / 2;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        float k0 = (float)kr[2 * u], k1 = (float)kr[2 * u + 1];
        rotate(k0, k1, cs_at(a, rc3[a], p0 + u));
        kp[4 * c8 + u][0] = (bf16)k0;
        kp[4 * c8 + u][1] = (bf16)k1;
        vp[4 * c8 + u][0] = vr[2 * u];
        vp[4 * c8 + u][1] = vr[2 * u + 1];
      }
    }
  }
  // product layout: lanes n, n + 32 serve key n (site halves hi)
  const int hi = lane >> 5, ql = lane & 31;
  const int pty = ql >> 3, ptx = ql & 7;
  f32x16 accK[2], accV[2];
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int e = 0; e < 16; e++) accK[t][e] = accV[t][e] = 0.f;

  for (int h = hk * g.G; h < (hk + 1) * g.G; h++) {
    __syncthreads();  // the previous head's stage is no longer read
    // the thread index, opaque within this head: the staging addresses and
    // slots are formed here rather than hoisted out of the head loop (spilled)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    // all loads first: raw q chunks, dO straight to LDS, per-site statistics
    bf16x8 qraw[RS];
#pragma unroll
    for (int r = 0; r < RS; r++) {
      const int e = min(tid + r * NT, NCK - 1);
      const int hs = e / CPS, ch = e % CPS;
      const int64_t off = ((bN + max(sSlot[hs], 0)) * g.H + h) * D + ch * 8;
      qraw[r] = *reinterpret_cast<const bf16x8 *>(q + off);
      __builtin_amdgcn_global_load_lds(dout + off, (lds_ptr)&sO[(wbase + r * NT) * 8], 16, 0, 0);
    }
    float st_g[RSL], st_l[RSL], st_d[RSL];
#pragma unroll
    for (int r = 0; r < RSL; r++) {
      const int hs = min(tid + r * NT, NH - 1);
      const int64_t srow = (bN + max(sSlot[hs], 0)) * g.H + h;
      st_g[r] = (float)gate[srow];
      st_l[r] = lse_l[srow];
      st_d[r] = delta_l[srow];
    }
#pragma unroll
    for (int r = 0; r < RS; r++) {
      const int e = tid + r * NT;
      const int ec = min(e, NCK - 1);
      const int hs = ec / CPS, ch = ec % CPS;
      const int qc3[3] = {hs / (HY * HX), (hs / HX) % HY, hs % HX};
      const int a = (ch * 8) / DA, p0 = ((ch * 8) % DA) / 2;
      bf16x8 qo;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        float x0 = (float)qraw[r][2 * u], x1 = (float)qraw[r][2 * u + 1];
        rotate(x0, x1, cs_at(a, qc3[a], p0 + u));
        qo[2 * u] = (bf16)(x0 * qscale);
        qo[2 * u + 1] = (bf16)(x1 * qscale);
      }
      *reinterpret_cast<bf16x8 *>(&sQ[e * 8]) = qo;
    }
#pragma unroll
    for (int r = 0; r < RSL; r++) {
      const int hs = tid + r * NT;
      if (hs < NH) {
        sOmg[hs] = 1.0f - 1.0f / (1.0f + expf(-st_g[r]));
        sL[hs] = st_l[r];
        sDl[hs] = st_d[r];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the key's corner index, opaque within this head (see k_bwd_local_kv_pair)
    int ksh = ((tz * HY) + ty) * HX + tx;
    asm volatile("" : "+v"(ksh));
    // logits (the query side's, bit for bit) and u_ij = <dO_i, v_j>; the
    // weights as bf16 triples (dx = -1, 0, +1) of each (dz, dy), packed as
    // the words (w-, w0) and (w+, 0); a key site without a token gets zeros
    uint32_t tK[9][2], tV[9][2];
#pragma unroll
    for (int r9 = 0; r9 < 9; r9++) {
      float pwr[3], dsr[3];
#pragma unroll
      for (int dx = 0; dx < 3; dx++) {
        const int kk = 3 * r9 + dx;
        const int hs = ksh + halo_from_corner(kk, HY, HX);
        const bf16x2 *qr = reinterpret_cast<const bf16x2 *>(sQ + hs * D + hh * DH);
        const bf16x2 *orr = reinterpret_cast<const bf16x2 *>(sO + hs * D + hh * DH);
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int jj = 0; jj < DH / 2; jj++) {
          a0 = __builtin_amdgcn_fdot2_f32_bf16(qr[jj], kp[jj], a0, false);
          a1 = __builtin_amdgcn_fdot2_f32_bf16(orr[jj], vp[jj], a1, false);
        }
        a0 = lane_sum<LPQ>(a0);
        a1 = lane_sum<LPQ>(a1);
        const bool valid = sSlot[hs] >= 0 && j >= 0;
        const float pr = valid ? __builtin_amdgcn_exp2f(a0 - sL[hs]) : 0.f;
        pwr[dx] = valid ? pr * sOmg[hs] : 0.f;
        dsr[dx] = valid ? pr * (sOmg[hs] * a1 - sDl[hs]) : 0.f;
        asm volatile("" ::: "memory");  // as on the query side
      }
      bf16x2 k0, k1, v0, v1;
      k0[0] = (bf16)dsr[0];
      k0[1] = (bf16)dsr[1];
      k1[0] = (bf16)dsr[2];
      k1[1] = (bf16)0.0f;
      v0[0] = (bf16)pwr[0];
      v0[1] = (bf16)pwr[1];
      v1[0] = (bf16)pwr[2];
      v1[1] = (bf16)0.0f;
      tK[r9][0] = __builtin_bit_cast(uint32_t, k0);
      tK[r9][1] = __builtin_bit_cast(uint32_t, k1);
      tV[r9][0] = __builtin_bit_cast(uint32_t, v0);
      tV[r9][1] = __builtin_bit_cast(uint32_t, v1);
    }
    // into the product layout: key n's words come from lane 2n
#pragma unroll
    for (int r9 = 0; r9 < 9; r9++)
#pragma unroll
      for (int w = 0; w < 2; w++) {
        tK[r9][w] = (uint32_t)__shfl((int)tK[r9][w], 2 * ql);
        tV[r9][w] = (uint32_t)__shfl((int)tV[r9][w], 2 * ql);
      }
    // Where this lane's weights sit in block kb4 of a plane: its window is
    // sites kappa0 = 16*kb4 + 8*hi .. +7 (kappa = y*10 + x of a halo plane);
    // the run of neighbour row dy starts at s_dy = (pty + 1 + dy)*10 + ptx,
    // and at most one run meets the window, at slot offset o in [-2, 7]
    // (for even o = 2m the pair itself in words m, m + 1; for odd o the
    // words (0, w-) and (w0, w+); zeros elsewhere).
    // the lane index, opaque within this head: the selectors and addresses
    // below are formed here rather than hoisted out of the head loop, where
    // they would spill
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lhi = ln >> 5, lq = ln & 31;
    const int grp = (ln >> 4) & 1, rq = ln & 3, re = (ln >> 2) & 3;
    const int abase = (tz * NPL + re) * D + 16 * grp + 4 * rq;  // elements
#pragma unroll
    for (int kb4 = 0; kb4 < 4; kb4++) {
      const int k0 = 16 * kb4 + 8 * lhi;
      const int sm = (lq >> 3) * 10 + (lq & 7);
      const int rel = k0 - sm + 7;
      const int di = rel >= 0 ? rel / 10 : -1;
      const bool ok = di >= 0 && di <= 2;
      const int o = sm + 10 * di - k0;
      const int m = ok ? (o >> 1) : -8;
      const bool odd = (o & 1) != 0;
      const uint32_t s0 = odd ? 0x01000C0Cu : 0x03020100u, s1 = odd ? 0x05040302u : 0x07060504u;
      uint32_t sel[4];
#pragma unroll
      for (int jd = 0; jd < 4; jd++) sel[jd] = jd == m ? s0 : (jd == m + 1 ? s1 : 0x0C0C0C0Cu);
#pragma unroll
      for (int dzi = 0; dzi < 3; dzi++) {
        // the even-packed triples of run di of plane dzi (selects between
        // constant indices: a run-time index would put the arrays in scratch)
        uint32_t xk[2], xv[2];
#pragma unroll
        for (int w = 0; w < 2; w++) {
          xk[w] = di == 0 ? tK[3 * dzi][w] : (di == 1 ? tK[3 * dzi + 1][w] : tK[3 * dzi + 2][w]);
          xv[w] = di == 0 ? tV[3 * dzi][w] : (di == 1 ? tV[3 * dzi + 1][w] : tV[3 * dzi + 2][w]);
        }
        uint32_t bk[4], bv[4];
#pragma unroll
        for (int jd = 0; jd < 4; jd++) {
          bk[jd] = __builtin_amdgcn_perm(xk[1], xk[0], sel[jd]);
          bv[jd] = __builtin_amdgcn_perm(xv[1], xv[0], sel[jd]);
        }
        bf16x8 bopK, bopV;
        __builtin_memcpy(&bopK, bk, 16);
        __builtin_memcpy(&bopV, bv, 16);
#pragma unroll
        for (int t = 0; t < 2; t++) {
          const int ad = abase + (dzi * NPL + k0) * D + 32 * t;
          const v4s ql4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(sQ + ad));
          const v4s qh4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(sQ + ad + 4 * D));
          const v4s ol4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(sO + ad));
          const v4s oh4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(sO + ad + 4 * D));
          bf16x8 aq, ao;
          __builtin_memcpy(&aq, &ql4, 8);
          __builtin_memcpy(reinterpret_cast<char *>(&aq) + 8, &qh4, 8);
          __builtin_memcpy(&ao, &ol4, 8);
          __builtin_memcpy(reinterpret_cast<char *>(&ao) + 8, &oh4, 8);
          accK[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bopK, accK[t], 0, 0, 0);
          accV[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, bopV, accV[t], 0, 0, 0);
        }
        // a compiler-only fence per plane: the next operands' LDS reads are
        // not all hoisted ahead, which would spill
        asm volatile("" ::: "memory");
      }
    }
  }
  // Lane (n, hi) holds channels 8*jj + 4*hi .. +3 of key n (tile jj / 4,
  // registers 4*(jj % 4) ..); the halves trade pieces (v_permlane32_swap)
  // so that each lane holds channels 16*mm + 8*hi .. +7, mm = 0, 1, 2.
  float okd[3][8], ovd[3][8];
#pragma unroll
  for (int mm = 0; mm < 3; mm++)
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int t0 = (2 * mm) / 4, r0 = 4 * ((2 * mm) % 4) + u;
      const int t1 = (2 * mm + 1) / 4, r1 = 4 * ((2 * mm + 1) % 4) + u;
      // elements copied out first: a bit cast applied straight to a vector
      // element subscript compiles to a cast of element 0
      const float k0 = accK[t0][r0], k1 = accK[t1][r1], v0 = accV[t0][r0], v1 = accV[t1][r1];
      const auto sk = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, k0),
                                                       __builtin_bit_cast(uint32_t, k1), false, false);
      const auto sv = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v0),
                                                       __builtin_bit_cast(uint32_t, v1), false, false);
      okd[mm][u] = __builtin_bit_cast(float, (uint32_t)sk[0]);
      okd[mm][4 + u] = __builtin_bit_cast(float, (uint32_t)sk[1]);
      ovd[mm][u] = __builtin_bit_cast(float, (uint32_t)sv[0]);
      ovd[mm][4 + u] = __builtin_bit_cast(float, (uint32_t)sv[1]);
    }
  // key n = ql of plane tz, in the product layout
  const int pj = sSlot[((tz + 1) * HY + (pty + 1)) * HX + (ptx + 1)];
  if (pj < 0) return;
  const int prc3[3] = {tz + 1, pty + 1, ptx + 1};
  // pooling transpose, then dk = R(c_j)^T dk~ (centre variant: its block part
  // goes through R(centre)^T instead)
  const int c3[3] = {z0 + tz, y0 + pty, x0 + ptx};
  const int mb = block_of(g, c3[0], c3[1], c3[2]);
  const int mz = mb / (g.My * g.Mx), my = (mb / g.Mx) % g.My, mx = mb % g.Mx;
  const int nm = min(g.bz, g.Z - mz * g.bz) * min(g.by, g.Y - my * g.by) * min(g.bx, g.X - mx * g.bx);
  const float inv_n = 1.0f / (float)nm;
  const int64_t prow = ((bN + pj) * g.Hkv + hk) * D;
  const float *gk = dks + (((int64_t)b * g.Hkv + hk) * g.M + mb) * D;
  const float *gv = dvs + (((int64_t)b * g.Hkv + hk) * g.M + mb) * D;
#pragma unroll
  for (int mm = 0; mm < 3; mm++) {
    const int d0 = 16 * mm + 8 * hi, a = mm, p0 = 4 * hi;  // axis chunk mm, its planes 4hi ..
    const f32x4 gk0 = *reinterpret_cast<const f32x4 *>(gk + d0);
    const f32x4 gk1 = *reinterpret_cast<const f32x4 *>(gk + d0 + 4);
    const f32x4 gv0 = *reinterpret_cast<const f32x4 *>(gv + d0);
    const f32x4 gv1 = *reinterpret_cast<const f32x4 *>(gv + d0 + 4);
    const float gkf[8] = {gk0[0], gk0[1], gk0[2], gk0[3], gk1[0], gk1[1], gk1[2], gk1[3]};
    const float gvf[8] = {gv0[0], gv0[1], gv0[2], gv0[3], gv1[0], gv1[1], gv1[2], gv1[3]};
    bf16x8 okv, ovv;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int c = 2 * u;
      float x0 = kLn2 * okd[mm][c], x1 = kLn2 * okd[mm][c + 1];  // s / (s log2 e)
      if (!CENTRE) {
        x0 += gkf[c] * inv_n;
        x1 += gkf[c + 1] * inv_n;
      }
      rotate_t(x0, x1, cs_at(a, prc3[a], p0 + u));
      if (CENTRE) {
        const int o = a == 0 ? mz * g.bz : (a == 1 ? my * g.by : mx * g.bx);
        const int ext = min(a == 0 ? g.bz : (a == 1 ? g.by : g.bx),
                            (a == 0 ? g.Z : (a == 1 ? g.Y : g.X)) - o);
        float2 t = rope_cs(tab, g, a, o + (ext - 1) / 2, p0 + u);
        if ((ext & 1) == 0) {
          const float2 hf = rope_half(tab, g, p0 + u);
          t = make_float2(t.x * hf.x - t.y * hf.y, t.y * hf.x + t.x * hf.y);
        }
        float y0 = gkf[c] * inv_n, y1 = gkf[c + 1] * inv_n;
        rotate_t(y0, y1, t);
        x0 += y0;
        x1 += y1;
      }
      okv[c] = (bf16)x0;
      okv[c + 1] = (bf16)x1;
      ovv[c] = (bf16)(ovd[mm][c] + gvf[c] * inv_n);
      ovv[c + 1] = (bf16)(ovd[mm][c + 1] + gvf[c + 1] * inv_n);
    }
    *reinterpret_cast<bf16x8 *>(dk + prow + d0) = okv;
    *reinterpret_cast<bf16x8 *>(dv + prow + d0) = ovv;
  }
}

// ---------------------------------------------------------------------------
namespace {
// The query side and the key side may use different boxes (KZ, KY, KX for
// the key side).
template <int D, int TZ, int TY, int TX, int KZ, int KY, int KX>
hipError_t run_local_bwd_pair(const Geo &g, const BwdArgs &a, hipStream_t s) {
  {
    const int ntz = (g.Z + TZ - 1) / TZ, nty = (g.Y + TY - 1) / TY, ntx = (g.X + TX - 1) / TX;
    const int nt = (D / 24) * TZ * TY * TX;
    // head dim 48: dq~ on the matrix cores
    auto qk = [] {
      if constexpr (D == 48 && TZ == 4 && TY == 4 && TX == 8)
        return k_bwd_local_q_tr48;
      else
        return k_bwd_local_q_pair<D, TZ, TY, TX>;
    }();
    hipLaunchKernelGGL(qk, dim3((unsigned)(g.B * ntz * nty * ntx * g.H)), dim3(nt), 0, s, g, a.geom,
                       static_cast<const bf16 *>(a.q), static_cast<const bf16 *>(a.k),
                       static_cast<const bf16 *>(a.v), static_cast<const bf16 *>(a.gate),
                       static_cast<const bf16 *>(a.dout), static_cast<const bf16 *>(a.oglob), a.dqg,
                       static_cast<bf16 *>(a.dq), static_cast<bf16 *>(a.dgate), a.lse_l, a.delta_l,
                       ntz, nty, ntx);
    if (hipError_t e = hipGetLastError()) return e;
  }
  const int ntz = (g.Z + KZ - 1) / KZ, nty = (g.Y + KY - 1) / KY, ntx = (g.X + KX - 1) / KX;
  const int nt = (D / 24) * KZ * KY * KX;
  const bool centre = (g.flags & PACK3D_SUMMARY_CENTRE) != 0;
  // head dim 48: the weighted sums on the matrix cores
  auto kv = [&] {
    if constexpr (D == 48 && KZ == 4 && KY == 4 && KX == 8)
      return centre ? k_bwd_local_kv_tr48<true> : k_bwd_local_kv_tr48<false>;
    else
      return centre ? k_bwd_local_kv_pair<D, KZ, KY, KX, true>
                    : k_bwd_local_kv_pair<D, KZ, KY, KX, false>;
  }();
  hipLaunchKernelGGL(kv, dim3((unsigned)(g.B * ntz * nty * ntx * g.Hkv)), dim3(nt), 0, s, g, a.geom,
                     static_cast<const bf16 *>(a.q), static_cast<const bf16 *>(a.k),
                     static_cast<const bf16 *>(a.v), static_cast<const bf16 *>(a.gate),
                     static_cast<const bf16 *>(a.dout), a.lse_l, a.delta_l, a.dks, a.dvs,
                     static_cast<bf16 *>(a.dk), static_cast<bf16 *>(a.dv), ntz, nty, ntx);
  return hipGetLastError();
}
}  // namespace

bool bwd_local_pair_supported(const Geo &g, int dtype) {
  return dtype == PACK3D_BF16 && (g.D == 48 || g.D == 96);
}

hipError_t launch_bwd_local_pair(const Geo &g, const BwdArgs &a, hipStream_t s) {
  if (g.D == 48) return run_local_bwd_pair<48, 4, 4, 8, 4, 4, 8>(g, a, s);
  // D = 96: the key side stages two halo tensors (q~ and dO); with 2 x 4 x 8
  // boxes (4 waves, 102 KB of LDS) one workgroup fits a CU, one wave per
  // SIMD; 4 x 4 x 8 boxes (8 waves, 152 KB) give two waves per SIMD
  return run_local_bwd_pair<96, 2, 4, 8, 4, 4, 8>(g, a, s);
}

}  // namespace pk
