/*
 * pack3d_oracle.c -- CPU oracle for the PACK3D local-global attention forward.
 *
 * TEST INFRASTRUCTURE. This file is the plain, slow, obviously correct
 * reference that the GPU library is checked against. Only the test suite,
 * the smoke entry point and the CPU-baseline leg of the benchmark may load
 * it. It shares no code, header, table or helper with the GPU library.
 *
 * Arithmetic is IEEE double throughout, in plain loops, with every reduction
 * taken in canonical coordinate order (neighbour offsets in a fixed order,
 * block members in within-block-slot order, summaries in block-id order).
 * Steps follow the method as the pages describe it (Geometry Matters in
 * Packed 3D Attention; "paper summary" = the arXiv 2610.38694 abstract page,
 * "project page" = the Pack3D site):
 *
 *   0. index          tokens carry integer grid coordinates; neighbourhoods
 *                     and blocks are defined on the lattice, never on memory
 *                     order (paper summary §B.1; project page Ch. 4, Prop. 2)
 *   1. axial RoPE     each head splits into rotation planes, one set per axis;
 *                     Q and K turn by their own (z,y,x), V is not rotated
 *                     (project page Ch. 3, Contract 3; paper summary §B.2)
 *   2. summaries      keys are rotated first, then mean-pooled per contiguous
 *                     3D block; values are pooled unrotated (project page
 *                     Ch. 3 "Rotate first, then pool"; paper summary §3.2, §B.5).
 *                     Variant: pool unrotated keys, rotate the mean once at
 *                     the block centre (paper summary §B.7, §B.8)
 *   3. local          exact softmax attention over the <=27 tokens of the
 *                     3x3x3 coordinate neighbourhood (project page Ch. 3,
 *                     Contract 1; paper summary §3.2, §3.5)
 *   4. global         every query attends to all block summaries (project
 *                     page Ch. 3, Contract 2; paper summary §3.5, §B.10)
 *   5. mix            a tokenwise gate combines the two branches (paper
 *                     summary §3.3, §4.4)
 *
 * Grouped key/value heads (GQA/MQA): keys, values and therefore the block
 * summaries exist per KV head (project page Ch. 3, Contract 2, which counts
 * summaries per KV head; paper summary §D.1, KV groups). With Hkv KV heads
 * and H query heads (H a multiple of Hkv), query head h reads KV head
 * floor(h / (H / Hkv)): consecutive query heads form a group. Hkv == H is
 * ordinary multi-head attention, Hkv == 1 multi-query attention.
 *
 * Readings taken where the pages are silent or garbled (the displayed
 * formulas did not survive): contiguous z|y|x channel chunks of D/3 per axis,
 * interleaved (2p, 2p+1) planes, theta_p = base^(-2p/(D/3)), integer 0-based
 * coordinates; neighbourhood = Chebyshev radius 1 including self, clipped at
 * the grid edge; scale 1/sqrt(D) in both branches; arithmetic mean pooling;
 * blocks aligned at coordinate 0, partial edge blocks average the members
 * present; no summary exclusion by default (exclusion of the query's own
 * block, or of every block meeting its clipped neighbourhood, is selectable);
 * gate g = sigmoid(G) per token and head, O = (1-g) O_loc + g O_glob.
 *
 * Parity pins (tests that fix this file to something other than itself):
 * index -> brute-force pair enumeration and closed-form counts; RoPE -> the
 * matrix exponential of the rotation generator; local -> dense masked SDPA in
 * float64; summaries -> the block-weighted displacement identity of §B.5;
 * global -> torch's scaled_dot_product_attention over the summaries; mix ->
 * saturated and neutral gates; whole operator -> bitwise packing equivariance.
 * The sequence-position RoPE control is pinned to the matrix exponential of
 * a 1-D rotation generator at the packed index, and by its failure to be
 * equivariant. Parity with the authors' own RoPE convention and numbers is
 * unpinned: no code, tables or worked numbers with all parameters are
 * printed on the pages.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t B, N, H, D;
  int32_t grid[3];   /* Z, Y, X (x fastest in raster order) */
  int32_t block[3];  /* bz, by, bx */
  double rope_base;  /* 10000 in every workload */
  double scale;      /* <= 0 selects 1/sqrt(D) */
  int32_t exclusion; /* 0 none, 1 own block, 2 blocks meeting the neighbourhood */
  int32_t Hkv;       /* key/value heads; 0 means H */
} ork_desc;

enum { ORK_OK = 0, ORK_ERR_ARG = -1, ORK_ERR_RANGE = -2, ORK_ERR_DUP = -3 };

int ork_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Number of key/value heads, and the KV head that query head h reads. */
static int kv_heads(const ork_desc *d) { return d->Hkv > 0 ? d->Hkv : d->H; }
static int kv_of(const ork_desc *d, int h) { return h / (d->H / kv_heads(d)); }

static double scale_of(const ork_desc *d) {
  return d->scale > 0 ? d->scale : 1.0 / sqrt((double)d->D);
}

static int64_t site_of(const ork_desc *d, int z, int y, int x) {
  return ((int64_t)z * d->grid[1] + y) * d->grid[2] + x;
}

static int blocks_along(const ork_desc *d, int a) {
  return (d->grid[a] + d->block[a] - 1) / d->block[a];
}

int ork_num_blocks(const ork_desc *d) {
  return blocks_along(d, 0) * blocks_along(d, 1) * blocks_along(d, 2);
}

/* Block id of a coordinate: blocks tile the lattice from coordinate 0, in
 * raster order of the block coordinate (floor(c / b)). */
static int block_id(const ork_desc *d, int z, int y, int x) {
  int mz = z / d->block[0], my = y / d->block[1], mx = x / d->block[2];
  return (mz * blocks_along(d, 1) + my) * blocks_along(d, 2) + mx;
}

/* Step 0. slot[site] = memory position of the token at that site; every
 * coordinate must lie in the grid and hit a distinct site. Also returns each
 * token's block id and its canonical slot inside the block, the metadata a
 * repack must carry (project page Ch. 4, Prop. 2). */
int ork_index(const ork_desc *d, const int32_t *coords, int32_t *slot,
              int32_t *blk, int32_t *rank) {
  int64_t S = (int64_t)d->grid[0] * d->grid[1] * d->grid[2];
  if (d->N <= 0 || S <= 0) return ORK_ERR_ARG;
  for (int64_t s = 0; s < S; s++) slot[s] = -1;
  for (int i = 0; i < d->N; i++) {
    int z = coords[3 * i], y = coords[3 * i + 1], x = coords[3 * i + 2];
    if (z < 0 || y < 0 || x < 0 || z >= d->grid[0] || y >= d->grid[1] || x >= d->grid[2])
      return ORK_ERR_RANGE;
    int64_t s = site_of(d, z, y, x);
    if (slot[s] != -1) return ORK_ERR_DUP;
    slot[s] = i;
    if (blk) blk[i] = block_id(d, z, y, x);
    if (rank) rank[i] = ((z % d->block[0]) * d->block[1] + (y % d->block[1])) * d->block[2] +
                        (x % d->block[2]);
  }
  return ORK_OK;
}

/* Neighbour k in 0..26 sits at offset (k/9 - 1, (k/3)%3 - 1, k%3 - 1); self is
 * k = 13. Off-grid offsets and empty sites give -1. */
static void offset_of(int k, int *dz, int *dy, int *dx) {
  *dz = k / 9 - 1;
  *dy = (k / 3) % 3 - 1;
  *dx = k % 3 - 1;
}

static int neighbour(const ork_desc *d, const int32_t *slot, const int32_t *c, int k) {
  int dz, dy, dx;
  offset_of(k, &dz, &dy, &dx);
  int z = c[0] + dz, y = c[1] + dy, x = c[2] + dx;
  if (z < 0 || y < 0 || x < 0 || z >= d->grid[0] || y >= d->grid[1] || x >= d->grid[2])
    return -1;
  return slot[site_of(d, z, y, x)];
}

void ork_neighbours(const ork_desc *d, const int32_t *coords, const int32_t *slot,
                    int32_t *nbr) {
  for (int i = 0; i < d->N; i++)
    for (int k = 0; k < 27; k++) nbr[27 * i + k] = neighbour(d, slot, coords + 3 * i, k);
}

/* Step 1. Axial RoPE at grid coordinates. Axis a in (z, y, x) owns channels
 * [a*D/3, (a+1)*D/3); plane p of that axis is the channel pair
 * (a*D/3 + 2p, a*D/3 + 2p + 1) with frequency theta_p = base^(-2p/(D/3)),
 * turned by angle c_a * theta_p. x, y: [B, N, H, D]. */
void ork_rope_axial(const ork_desc *d, const int32_t *coords, const double *x, double *y) {
  const int D = d->D, da = D / 3, P = da / 2;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < (int64_t)d->B * d->N * d->H; row++) {
    int i = (int)((row / d->H) % d->N);
    const double *xr = x + row * D;
    double *yr = y + row * D;
    for (int a = 0; a < 3; a++) {
      for (int p = 0; p < P; p++) {
        double theta = pow(d->rope_base, -2.0 * p / (double)da);
        double phi = (double)coords[3 * i + a] * theta;
        double cs = cos(phi), sn = sin(phi);
        int c0 = a * da + 2 * p;
        double x0 = xr[c0], x1 = xr[c0 + 1];
        yr[c0] = x0 * cs - x1 * sn;
        yr[c0 + 1] = x0 * sn + x1 * cs;
      }
    }
  }
}

/* Control: the same rotation indexed by packed memory position i over all D
 * channels (theta_p = base^(-2p/D)), i.e. RoPE at the sequence index, which
 * the pages show is not packing-equivariant (paper summary §B.4). */
void ork_rope_sequence(const ork_desc *d, const double *x, double *y) {
  const int D = d->D, P = D / 2;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < (int64_t)d->B * d->N * d->H; row++) {
    int i = (int)((row / d->H) % d->N);
    const double *xr = x + row * D;
    double *yr = y + row * D;
    for (int p = 0; p < P; p++) {
      double theta = pow(d->rope_base, -2.0 * p / (double)D);
      double phi = (double)i * theta;
      double cs = cos(phi), sn = sin(phi);
      double x0 = xr[2 * p], x1 = xr[2 * p + 1];
      yr[2 * p] = x0 * cs - x1 * sn;
      yr[2 * p + 1] = x0 * sn + x1 * cs;
    }
  }
}

/* Step 2. Rotate-then-pool block summaries. For block m, members are visited
 * in canonical within-block slot order r = ((z%bz)*by + y%by)*bx + x%bx; the
 * summary key is the mean of the members' ROTATED keys, the summary value the
 * mean of their values. Sites that are off-grid (partial edge blocks) or
 * empty do not count. Summaries exist per KV head. kr, v: [B, N, Hkv, D];
 * ks, vs: [B, Hkv, M, D]. */
void ork_summaries(const ork_desc *d, const int32_t *slot, const double *kr, const double *v,
                   double *ks, double *vs) {
  const int D = d->D, H = kv_heads(d), M = ork_num_blocks(d);
  const int My = blocks_along(d, 1), Mx = blocks_along(d, 2);
  const int bz = d->block[0], by = d->block[1], bx = d->block[2];
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < d->B; b++) {
    for (int m = 0; m < M; m++) {
      int oz = (m / (My * Mx)) * bz, oy = ((m / Mx) % My) * by, ox = (m % Mx) * bx;
      for (int h = 0; h < H; h++) {
        double *ko = ks + (((int64_t)b * H + h) * M + m) * D;
        double *vo = vs + (((int64_t)b * H + h) * M + m) * D;
        for (int c = 0; c < D; c++) ko[c] = vo[c] = 0.0;
        int count = 0;
        for (int r = 0; r < bz * by * bx; r++) {
          int z = oz + r / (by * bx), y = oy + (r / bx) % by, x = ox + r % bx;
          if (z >= d->grid[0] || y >= d->grid[1] || x >= d->grid[2]) continue;
          int j = slot[site_of(d, z, y, x)];
          if (j < 0) continue;
          const double *kj = kr + (((int64_t)b * d->N + j) * H + h) * D;
          const double *vj = v + (((int64_t)b * d->N + j) * H + h) * D;
          for (int c = 0; c < D; c++) {
            ko[c] += kj[c];
            vo[c] += vj[c];
          }
          count++;
        }
        if (count > 0)
          for (int c = 0; c < D; c++) {
            ko[c] /= count;
            vo[c] /= count;
          }
      }
    }
  }
}

/* Block centre of block m: origin + (extent - 1) / 2 per axis, the extent
 * clipped at the grid edge (a half-integer coordinate for an even extent). */
static void block_centre(const ork_desc *d, int m, double *centre) {
  const int My = blocks_along(d, 1), Mx = blocks_along(d, 2);
  const int o[3] = {(m / (My * Mx)) * d->block[0], ((m / Mx) % My) * d->block[1],
                    (m % Mx) * d->block[2]};
  for (int a = 0; a < 3; a++) {
    int extent = d->grid[a] - o[a] < d->block[a] ? d->grid[a] - o[a] : d->block[a];
    centre[a] = o[a] + 0.5 * (extent - 1);
  }
}

/* Summary-centre variant (paper summary §B.7, §B.8; project page Ch. 3, the
 * cheaper summary that pools unrotated keys and rotates the result once at a
 * representative coordinate). The keys k are the unrotated inputs; each
 * block's mean key is rotated at the block centre, origin + (extent - 1) / 2
 * along each axis, the extent clipped at the grid edge (a half-integer
 * coordinate for an even extent). Values are pooled as in ork_summaries. */
void ork_summaries_centre(const ork_desc *d, const int32_t *slot, const double *k,
                          const double *v, double *ks, double *vs) {
  ork_summaries(d, slot, k, v, ks, vs); /* plain means of the unrotated keys */
  const int D = d->D, H = kv_heads(d), M = ork_num_blocks(d), da = D / 3, P = da / 2;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < d->B; b++) {
    for (int m = 0; m < M; m++) {
      double centre[3];
      block_centre(d, m, centre);
      for (int h = 0; h < H; h++) {
        double *ko = ks + (((int64_t)b * H + h) * M + m) * D;
        for (int a = 0; a < 3; a++) {
          for (int p = 0; p < P; p++) {
            double theta = pow(d->rope_base, -2.0 * (double)p / (double)da);
            double phi = centre[a] * theta;
            double cs = cos(phi), sn = sin(phi);
            const int first = a * da + 2 * p; /* channels (first, first + 1) */
            double x0 = ko[first], x1 = ko[first + 1];
            ko[first] = x0 * cs - x1 * sn;
            ko[first + 1] = x0 * sn + x1 * cs;
          }
        }
      }
    }
  }
}

static double dot(const double *a, const double *b, int n) {
  double s = 0.0;
  for (int c = 0; c < n; c++) s += a[c] * b[c];
  return s;
}

/* Step 3. Exact local attention for the selected query tokens rows[0..nrows)
 * (rows == NULL: all N). Logits s*<q~_i, k~_j> over the valid neighbours in
 * offset order, softmax with the maximum subtracted, then the weighted sum of
 * the neighbours' (unrotated) values. Self is always valid, so the set is
 * never empty. Query head h reads KV head kv_of(h). qr: [B, N, H, D];
 * kr, v: [B, N, Hkv, D]; out: [B, nrows, H, D]. */
void ork_local(const ork_desc *d, const int32_t *coords, const int32_t *slot, const double *qr,
               const double *kr, const double *v, const int32_t *rows, int nrows, double *out) {
  const int D = d->D, H = d->H, Hk = kv_heads(d);
  const double s = scale_of(d);
  if (!rows) nrows = d->N;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < d->B; b++) {
    for (int t = 0; t < nrows; t++) {
      int i = rows ? rows[t] : t;
      int nb[27];
      for (int k = 0; k < 27; k++) nb[k] = neighbour(d, slot, coords + 3 * i, k);
      for (int h = 0; h < H; h++) {
        const double *q = qr + (((int64_t)b * d->N + i) * H + h) * D;
        double logit[27], mx = -INFINITY;
        for (int k = 0; k < 27; k++) {
          if (nb[k] < 0) continue;
          logit[k] = s * dot(q, kr + (((int64_t)b * d->N + nb[k]) * Hk + kv_of(d, h)) * D, D);
          if (logit[k] > mx) mx = logit[k];
        }
        double den = 0.0;
        for (int k = 0; k < 27; k++)
          if (nb[k] >= 0) den += exp(logit[k] - mx);
        double *o = out + (((int64_t)b * nrows + t) * H + h) * D;
        for (int c = 0; c < D; c++) o[c] = 0.0;
        for (int k = 0; k < 27; k++) {
          if (nb[k] < 0) continue;
          double p = exp(logit[k] - mx) / den;
          const double *vj = v + (((int64_t)b * d->N + nb[k]) * Hk + kv_of(d, h)) * D;
          for (int c = 0; c < D; c++) o[c] += p * vj[c];
        }
      }
    }
  }
}

/* Whether summary m is withheld from query coordinate c under the selected
 * exclusion reading (0: none). */
static int excluded(const ork_desc *d, const int32_t *c, int m) {
  if (d->exclusion == 0) return 0;
  if (d->exclusion == 1) return m == block_id(d, c[0], c[1], c[2]);
  for (int k = 0; k < 27; k++) {
    int dz, dy, dx;
    offset_of(k, &dz, &dy, &dx);
    int z = c[0] + dz, y = c[1] + dy, x = c[2] + dx;
    if (z < 0 || y < 0 || x < 0 || z >= d->grid[0] || y >= d->grid[1] || x >= d->grid[2])
      continue;
    if (block_id(d, z, y, x) == m) return 1;
  }
  return 0;
}

/* Step 4. Query-to-summary attention: logits s*<q~_i, ks_m> over every
 * summary m (minus the excluded ones) in block-id order, softmax with the
 * maximum subtracted, weighted sum of the summary values. If every summary is
 * excluded the branch output is zero. Query head h reads the summaries of KV
 * head kv_of(h). qr: [B, N, H, D]; ks, vs: [B, Hkv, M, D]; out: [B, nrows, H, D]. */
void ork_global(const ork_desc *d, const int32_t *coords, const double *qr, const double *ks,
                const double *vs, const int32_t *rows, int nrows, double *out) {
  const int D = d->D, H = d->H, Hk = kv_heads(d), M = ork_num_blocks(d);
  const double s = scale_of(d);
  if (!rows) nrows = d->N;
#pragma omp parallel
  {
    double *logit = (double *)malloc(sizeof(double) * (size_t)M);
#pragma omp for collapse(2) schedule(static)
    for (int b = 0; b < d->B; b++) {
      for (int t = 0; t < nrows; t++) {
        int i = rows ? rows[t] : t;
        for (int h = 0; h < H; h++) {
          const double *q = qr + (((int64_t)b * d->N + i) * H + h) * D;
          double mx = -INFINITY;
          for (int m = 0; m < M; m++) {
            if (excluded(d, coords + 3 * i, m)) {
              logit[m] = -INFINITY;
              continue;
            }
            logit[m] = s * dot(q, ks + (((int64_t)b * Hk + kv_of(d, h)) * M + m) * D, D);
            if (logit[m] > mx) mx = logit[m];
          }
          double *o = out + (((int64_t)b * nrows + t) * H + h) * D;
          for (int c = 0; c < D; c++) o[c] = 0.0;
          if (mx == -INFINITY) continue;
          double den = 0.0;
          for (int m = 0; m < M; m++)
            if (logit[m] != -INFINITY) den += exp(logit[m] - mx);
          for (int m = 0; m < M; m++) {
            if (logit[m] == -INFINITY) continue;
            double p = exp(logit[m] - mx) / den;
            const double *vm = vs + (((int64_t)b * Hk + kv_of(d, h)) * M + m) * D;
            for (int c = 0; c < D; c++) o[c] += p * vm[c];
          }
        }
      }
    }
    free(logit);
  }
}

/* Step 5. Tokenwise mix: g = 1/(1+exp(-G)), O = (1-g) O_loc + g O_glob.
 * gate: [B, N, H] indexed at rows; oloc, oglob, out: [B, nrows, H, D]. */
void ork_mix(const ork_desc *d, const double *gate, const double *oloc, const double *oglob,
             const int32_t *rows, int nrows, double *out) {
  const int D = d->D, H = d->H;
  if (!rows) nrows = d->N;
  for (int b = 0; b < d->B; b++)
    for (int t = 0; t < nrows; t++) {
      int i = rows ? rows[t] : t;
      for (int h = 0; h < H; h++) {
        double g = 1.0 / (1.0 + exp(-gate[((int64_t)b * d->N + i) * H + h]));
        int64_t base = (((int64_t)b * nrows + t) * H + h) * D;
        for (int c = 0; c < D; c++) out[base + c] = (1.0 - g) * oloc[base + c] + g * oglob[base + c];
      }
    }
}

/* ------------------------------------------------------------------------
 * Backward of the whole operator: the gradients of a scalar loss with
 * respect to q, k, v and the gate logits, given dout = dL/dO. The pages'
 * operator is trained end to end and its backward follows the forward's
 * access pattern (paper summary §1, §3.4); the steps below are the chain
 * rule through steps 5, 4, 3, 2 and 1 in reverse order, each one the plain
 * derivative of the forward step it undoes:
 *
 *   mix     g = sigmoid(G): dG = g (1 - g) <dO, O_glob - O_loc>,
 *           dO_loc = (1 - g) dO, dO_glob = g dO
 *   softmax attention (local over the neighbours, global over the allowed
 *           summaries), P = softmax(s <q~, k>), O = sum P v:
 *           dP_j = <dO, v_j>, Delta = sum_j P_j dP_j,
 *           dS_j = P_j (dP_j - Delta), dq~ += s sum_j dS_j k_j,
 *           dk_j += s dS_j q~, dv_j += P_j dO
 *   pooling mean over the n_m members present: each member receives
 *           dk_sum / n_m and dv_sum / n_m (token summaries: the rotated key
 *           k~_j; centre summaries: R(centre)^T dk_sum / n_m on the
 *           unrotated key)
 *   RoPE    x~ = R(c) x is orthogonal: dx = R(c)^T dx~
 *
 * With grouped KV heads the key and value gradients of a KV head sum over
 * its group of query heads. Inputs as in the forward (q [B,N,H,D],
 * k, v [B,N,Hkv,D], gate [B,N,H]); dout, dq [B,N,H,D]; dk, dv [B,N,Hkv,D];
 * dgate [B,N,H]. centre selects the summary-centre variant. Returns
 * ORK_OK, or an index error (off-grid / duplicate coordinate).
 */

/* x~ = R(c) x (sign +1) or x = R(c)^T x~ (sign -1) on one [D] row at the
 * real coordinate c (z, y, x). */
static void rotate_row(const ork_desc *d, const double *c, const double *x, double *y, int sign) {
  const int D = d->D, da = D / 3, P = da / 2;
  for (int a = 0; a < 3; a++) {
    for (int p = 0; p < P; p++) {
      const double theta = pow(d->rope_base, -(2.0 * p) / (double)da);
      const double cs = cos(c[a] * theta), sn = sign * sin(c[a] * theta);
      const int ch = 2 * p + a * da; /* plane p of axis a: channels ch, ch + 1 */
      const double x0 = x[ch], x1 = x[ch + 1];
      y[ch] = x0 * cs - x1 * sn;
      y[ch + 1] = x0 * sn + x1 * cs;
    }
  }
}

static void rotate_rows(const ork_desc *d, const int32_t *coords, int heads, const double *x,
                        double *y, int sign) {
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < (int64_t)d->B * d->N * heads; row++) {
    int i = (int)((row / heads) % d->N);
    double c[3] = {coords[3 * i], coords[3 * i + 1], coords[3 * i + 2]};
    rotate_row(d, c, x + row * d->D, y + row * d->D, sign);
  }
}

int ork_backward(const ork_desc *d, const int32_t *coords, const double *q, const double *k,
                 const double *v, const double *gate, const double *dout, int centre,
                 double *dq, double *dk, double *dv, double *dgate) {
  const int B = d->B, N = d->N, H = d->H, Hk = kv_heads(d), D = d->D, M = ork_num_blocks(d);
  const int G = H / Hk;
  const double s = scale_of(d);
  const int64_t nq = (int64_t)B * N * H * D, nk = (int64_t)B * N * Hk * D,
                ns = (int64_t)B * Hk * M * D;
  int64_t S = (int64_t)d->grid[0] * d->grid[1] * d->grid[2];
  int32_t *slot = malloc(sizeof(int32_t) * S);
  int rc = ork_index(d, coords, slot, NULL, NULL);
  if (rc != ORK_OK) {
    free(slot);
    return rc;
  }
  double *qr = malloc(sizeof(double) * nq), *kr = malloc(sizeof(double) * nk);
  double *ks = malloc(sizeof(double) * ns), *vs = malloc(sizeof(double) * ns);
  double *ol = malloc(sizeof(double) * nq), *og = malloc(sizeof(double) * nq);
  double *dol = malloc(sizeof(double) * nq), *dog = malloc(sizeof(double) * nq);
  double *dqr = calloc(nq, sizeof(double)), *dkr = calloc(nk, sizeof(double));
  double *dks = calloc(ns, sizeof(double)), *dvs = calloc(ns, sizeof(double));

  /* forward values the derivatives need */
  rotate_rows(d, coords, H, q, qr, +1);
  rotate_rows(d, coords, Hk, k, kr, +1);
  if (centre)
    ork_summaries_centre(d, slot, k, v, ks, vs);
  else
    ork_summaries(d, slot, kr, v, ks, vs);
  ork_local(d, coords, slot, qr, kr, v, NULL, 0, ol);
  ork_global(d, coords, qr, ks, vs, NULL, 0, og);

  /* mix */
  for (int64_t r = 0; r < (int64_t)B * N * H; r++) {
    double g = 1.0 / (1.0 + exp(-gate[r]));
    const double *o0 = ol + r * D, *o1 = og + r * D, *dor = dout + r * D;
    double acc = 0.0;
    for (int c = 0; c < D; c++) {
      acc += dor[c] * (o1[c] - o0[c]);
      dol[r * D + c] = (1.0 - g) * dor[c];
      dog[r * D + c] = g * dor[c];
    }
    dgate[r] = g * (1.0 - g) * acc;
  }
  for (int64_t e = 0; e < nk; e++) dv[e] = 0.0;

  /* local attention; each (b, KV head) owns its key and value gradients */
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; b++) {
    for (int hk = 0; hk < Hk; hk++) {
      for (int h = hk * G; h < (hk + 1) * G; h++) {
        for (int i = 0; i < N; i++) {
          int nb[27];
          double logit[27], p[27], dp[27], mx = -INFINITY, den = 0.0, delta = 0.0;
          const double *qi = qr + (((int64_t)b * N + i) * H + h) * D;
          const double *doi = dol + (((int64_t)b * N + i) * H + h) * D;
          double *dqi = dqr + (((int64_t)b * N + i) * H + h) * D;
          for (int n = 0; n < 27; n++) {
            nb[n] = neighbour(d, slot, coords + 3 * i, n);
            if (nb[n] < 0) continue;
            logit[n] = s * dot(qi, kr + (((int64_t)b * N + nb[n]) * Hk + hk) * D, D);
            if (logit[n] > mx) mx = logit[n];
          }
          for (int n = 0; n < 27; n++)
            if (nb[n] >= 0) den += exp(logit[n] - mx);
          for (int n = 0; n < 27; n++) {
            if (nb[n] < 0) continue;
            p[n] = exp(logit[n] - mx) / den;
            dp[n] = dot(doi, v + (((int64_t)b * N + nb[n]) * Hk + hk) * D, D);
            delta += p[n] * dp[n];
          }
          for (int n = 0; n < 27; n++) {
            if (nb[n] < 0) continue;
            const double ds = p[n] * (dp[n] - delta);
            const int64_t jo = (((int64_t)b * N + nb[n]) * Hk + hk) * D;
            for (int c = 0; c < D; c++) {
              dqi[c] += s * ds * kr[jo + c];
              dkr[jo + c] += s * ds * qi[c];
              dv[jo + c] += p[n] * doi[c];
            }
          }
        }
      }
    }
  }

  /* global attention over the summaries */
#pragma omp parallel
  {
    double *logit = malloc(sizeof(double) * (size_t)M);
#pragma omp for collapse(2) schedule(static)
    for (int b = 0; b < B; b++) {
      for (int hk = 0; hk < Hk; hk++) {
        for (int h = hk * G; h < (hk + 1) * G; h++) {
          for (int i = 0; i < N; i++) {
            const double *qi = qr + (((int64_t)b * N + i) * H + h) * D;
            const double *doi = dog + (((int64_t)b * N + i) * H + h) * D;
            double *dqi = dqr + (((int64_t)b * N + i) * H + h) * D;
            const int64_t sb = ((int64_t)b * Hk + hk) * M;
            double mx = -INFINITY, den = 0.0, delta = 0.0;
            for (int m = 0; m < M; m++) {
              logit[m] = excluded(d, coords + 3 * i, m) ? -INFINITY
                                                         : s * dot(qi, ks + (sb + m) * D, D);
              if (logit[m] > mx) mx = logit[m];
            }
            if (mx == -INFINITY) continue; /* every summary excluded: O_glob = 0 */
            for (int m = 0; m < M; m++)
              if (logit[m] != -INFINITY) den += exp(logit[m] - mx);
            for (int m = 0; m < M; m++)
              if (logit[m] != -INFINITY)
                delta += exp(logit[m] - mx) / den * dot(doi, vs + (sb + m) * D, D);
            for (int m = 0; m < M; m++) {
              if (logit[m] == -INFINITY) continue;
              const double pm = exp(logit[m] - mx) / den;
              const double dt = pm * (dot(doi, vs + (sb + m) * D, D) - delta);
              for (int c = 0; c < D; c++) {
                dqi[c] += s * dt * ks[(sb + m) * D + c];
                dks[(sb + m) * D + c] += s * dt * qi[c];
                dvs[(sb + m) * D + c] += pm * doi[c];
              }
            }
          }
        }
      }
    }
    free(logit);
  }

  /* pooling: each member present gets the block's gradient over n_m */
  const int My = blocks_along(d, 1), Mx = blocks_along(d, 2);
  const int bz = d->block[0], by = d->block[1], bx = d->block[2];
  double *dkc = centre ? calloc(nk, sizeof(double)) : NULL; /* unrotated-key part */
  int *members = malloc(sizeof(int) * (size_t)bz * by * bx);
  double *gku = malloc(sizeof(double) * D);
  for (int b = 0; b < B; b++) {
    for (int m = 0; m < M; m++) {
      const int oz = bz * (m / (My * Mx)), oy = by * ((m / Mx) % My), ox = bx * (m % Mx);
      int count = 0;
      for (int r = 0; r < bz * by * bx; r++) {
        int z = oz + r / (by * bx), y = oy + (r / bx) % by, x = ox + r % bx;
        if (z >= d->grid[0] || y >= d->grid[1] || x >= d->grid[2]) continue;
        int j = slot[site_of(d, z, y, x)];
        if (j >= 0) members[count++] = j;
      }
      if (count == 0) continue;
      double cm[3];
      block_centre(d, m, cm);
      for (int hk = 0; hk < Hk; hk++) {
        const double *gk = dks + (((int64_t)b * Hk + hk) * M + m) * D;
        const double *gv = dvs + (((int64_t)b * Hk + hk) * M + m) * D;
        if (centre) rotate_row(d, cm, gk, gku, -1);
        for (int t = 0; t < count; t++) {
          const int64_t jo = (((int64_t)b * N + members[t]) * Hk + hk) * D;
          for (int c = 0; c < D; c++) {
            if (centre)
              dkc[jo + c] += gku[c] / count;
            else
              dkr[jo + c] += gk[c] / count;
            dv[jo + c] += gv[c] / count;
          }
        }
      }
    }
  }
  free(members);
  free(gku);

  /* RoPE: back through the orthogonal rotations */
  rotate_rows(d, coords, H, dqr, dq, -1);
  rotate_rows(d, coords, Hk, dkr, dk, -1);
  if (centre)
    for (int64_t e = 0; e < nk; e++) dk[e] += dkc[e];

  free(slot);
  free(qr);
  free(kr);
  free(ks);
  free(vs);
  free(ol);
  free(og);
  free(dol);
  free(dog);
  free(dqr);
  free(dkr);
  free(dks);
  free(dvs);
  free(dkc);
  return ORK_OK;
}
