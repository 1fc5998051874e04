// Geometry metadata: slot map, coordinate checks, RoPE table and the optional
// neighbour / block / within-block-slot exports. Tokens are indexed by their
// grid coordinate, never by memory order (Geometry Matters in Packed 3D
// Attention, paper summary §B.1; project page Ch. 4, Prop. 2).
#include "launch.hpp"

namespace pk {

// Clears the status word and slot map and fills the RoPE table: one row per
// grid coordinate of each axis, then one row of half-angles theta_p / 2 (a
// block centre of even extent sits half-way between two coordinates).
__global__ void k_geom_init(Geo g, int32_t *status, int32_t *slot, float2 *tab) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t S = (int64_t)g.Z * g.Y * g.X;
  if (t == 0) status[0] = 0;
  if (t < 16) status[kZeroOff / 4 + t] = 0;  // the header's zero bytes
  if (t < S) slot[t] = -1;
  const int rows = g.Z + g.Y + g.X;
  int64_t T = (int64_t)(rows + 1) * g.P;
  if (t < T) {
    int row = (int)(t / g.P), p = (int)(t % g.P);
    int c = row < g.Z ? row : (row < g.Z + g.Y ? row - g.Z : row - g.Z - g.Y);
    tab[t] = row < rows ? rope_cs_direct(g.rope_base, g.D, c, p)
                        : rope_cs_real(g.rope_base, g.D, 0.5, p);
  }
}

// slot[site(c_i)] = i; bit 0 of the status word marks an off-grid
// coordinate, bit 1 a site claimed twice. A site claimed by several tokens
// keeps the lowest memory index whatever order the claims arrive in: the
// empty slot (-1) is the largest value as an unsigned word, so an unsigned
// atomic minimum takes the first claim and every lower index after it.
__global__ void k_geom_scatter(Geo g, const int32_t *coords, int32_t *status, int32_t *slot) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= g.N) return;
  int z = coords[3 * (int64_t)i], y = coords[3 * (int64_t)i + 1], x = coords[3 * (int64_t)i + 2];
  if (z < 0 || y < 0 || x < 0 || z >= g.Z || y >= g.Y || x >= g.X) {
    atomicOr(status, 1);
    return;
  }
  unsigned old = atomicMin(reinterpret_cast<unsigned *>(&slot[site_of(g, z, y, x)]), (unsigned)i);
  if (old != 0xFFFFFFFFu) atomicOr(status, 2);
}

__global__ void k_geom_export(Geo g, const int32_t *coords, const int32_t *slot, int32_t *nbr,
                              int32_t *blk, int32_t *rank) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= g.N) return;
  int z = coords[3 * (int64_t)i], y = coords[3 * (int64_t)i + 1], x = coords[3 * (int64_t)i + 2];
  bool in = !(z < 0 || y < 0 || x < 0 || z >= g.Z || y >= g.Y || x >= g.X);
  if (blk) blk[i] = in ? block_of(g, z, y, x) : -1;
  if (rank) rank[i] = in ? ((z % g.bz) * g.by + (y % g.by)) * g.bx + (x % g.bx) : -1;
  if (nbr) {
    for (int k = 0; k < 27; k++) {
      int zz = z + k / 9 - 1, yy = y + (k / 3) % 3 - 1, xx = x + k % 3 - 1;
      bool ok = in && zz >= 0 && yy >= 0 && xx >= 0 && zz < g.Z && yy < g.Y && xx < g.X;
      nbr[(int64_t)i * 27 + k] = ok ? slot_get(g, slot, site_of(g, zz, yy, xx)) : -1;
    }
  }
}

// Zeroes, for every token that takes no part (coordinate off the grid, or a
// site that went to a lower memory index), its row in each of up to four
// [B, N, len] tensors of es-byte elements (a null pointer is skipped). The
// kernels that reach tokens through the slot map never write those rows.
__global__ void k_zero_absent(Geo g, const void *geom, const int32_t *__restrict__ coords,
                              char *r0, char *r1, char *r2, char *r3, int b0, int b1, int b2,
                              int b3) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)g.B * g.N) return;
  const int i = (int)(t % g.N);
  const int z = coords[3 * (int64_t)i], y = coords[3 * (int64_t)i + 1], x = coords[3 * (int64_t)i + 2];
  if (takes_part(g, slot_map(geom, g), i, z, y, x)) return;
  char *rows[4] = {r0, r1, r2, r3};
  const int bytes[4] = {b0, b1, b2, b3};
  for (int k = 0; k < 4; k++)
    if (rows[k])
      for (int e = 0; e < bytes[k]; e++) rows[k][t * bytes[k] + e] = 0;
}

hipError_t launch_zero_absent(const Geo &g, int es, const void *geom, const int32_t *coords,
                              void *const *rows, const int *len, hipStream_t s) {
  const int64_t n = (int64_t)g.B * g.N;
  hipLaunchKernelGGL(k_zero_absent, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, geom,
                     coords, static_cast<char *>(rows[0]), static_cast<char *>(rows[1]),
                     static_cast<char *>(rows[2]), static_cast<char *>(rows[3]), len[0] * es,
                     len[1] * es, len[2] * es, len[3] * es);
  return hipGetLastError();
}

hipError_t launch_index(const Geo &g, const int32_t *coords, void *geom, int32_t *nbr,
                        int32_t *blk, int32_t *rank, hipStream_t s) {
  char *base = static_cast<char *>(geom);
  int32_t *status = reinterpret_cast<int32_t *>(base);
  int32_t *slot = reinterpret_cast<int32_t *>(base + g.slot_off);
  float2 *tab = reinterpret_cast<float2 *>(base + g.table_off);
  int64_t S = (int64_t)g.Z * g.Y * g.X;
  int64_t T = (int64_t)(g.Z + g.Y + g.X + 1) * g.P;
  int64_t n = S > T ? S : T;
  const int TB = 256;
  hipLaunchKernelGGL(k_geom_init, dim3((unsigned)((n + TB - 1) / TB)), dim3(TB), 0, s, g, status,
                     slot, tab);
  hipLaunchKernelGGL(k_geom_scatter, dim3((unsigned)((g.N + TB - 1) / TB)), dim3(TB), 0, s, g,
                     coords, status, slot);
  if (nbr || blk || rank)
    hipLaunchKernelGGL(k_geom_export, dim3((unsigned)((g.N + TB - 1) / TB)), dim3(TB), 0, s, g,
                       coords, slot, nbr, blk, rank);
  return hipGetLastError();
}

}  // namespace pk
