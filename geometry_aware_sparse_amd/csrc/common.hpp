// Device-side helpers shared by the PACK3D gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pack3d.h"

namespace pk {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// LDS destination of a direct global->LDS load
typedef __attribute__((address_space(3))) void *lds_ptr;

// Raw buffer resource over [p, p + bytes) (32-bit data format, no swizzle),
// for buffer loads into LDS. The tiled matrix-core kernels stage through
// buffer loads rather than flat global->LDS loads: while a flat LDS load is
// in flight the compiler cannot count LDS reads in order, and waits for all
// of them before any use of one; with buffer loads it waits for each read
// alone. Offsets are 32-bit bytes, so callers check that a slice fits.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}

// Problem geometry, derived once on the host from pack3d_desc and passed to
// kernels by value.
struct Geo {
  int B, N, H, D;
  int Hkv;        // key/value heads; query head h reads KV head h / G
  int G;          // query heads per KV head, H / Hkv
  int Z, Y, X;
  int bz, by, bx;
  int Mz, My, Mx;
  int M;          // number of summaries
  int P;          // rotation planes per axis = D / 6
  int vol;        // bz * by * bx
  float scale;    // softmax scale
  float rope_base;
  int excl;       // pack3d_exclusion
  unsigned flags; // pack3d_desc flags
  // geometry buffer offsets (bytes)
  int64_t slot_off, table_off;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Byte offset, in the geometry buffer's header, of 64 zero bytes.
constexpr int kZeroOff = 64;

__device__ __forceinline__ const int32_t *slot_map(const void *geom, const Geo &g) {
  return reinterpret_cast<const int32_t *>(static_cast<const char *>(geom) + g.slot_off);
}
__device__ __forceinline__ const float2 *rope_table(const void *geom, const Geo &g) {
  return reinterpret_cast<const float2 *>(static_cast<const char *>(geom) + g.table_off);
}
// (cos, sin) for axis a at coordinate c, plane p.
__device__ __forceinline__ float2 rope_cs(const float2 *tab, const Geo &g, int a, int c, int p) {
  int start = a == 0 ? 0 : (a == 1 ? g.Z : g.Z + g.Y);
  return tab[(int64_t)(start + c) * g.P + p];
}
// (cos, sin) of half of plane p's angle per unit step: the table's last row.
__device__ __forceinline__ float2 rope_half(const float2 *tab, const Geo &g, int p) {
  return tab[(int64_t)(g.Z + g.Y + g.X) * g.P + p];
}
// The same value computed directly: angle c * base^(-2p/(D/3)) in double,
// cos and sin in double, rounded to fp32.
__device__ __forceinline__ float2 rope_cs_direct(float base, int D, int c, int p) {
  double theta = pow((double)base, -2.0 * (double)p / (double)(D / 3));
  double phi = (double)c * theta;
  double s, co;
  sincos(phi, &s, &co);
  return make_float2((float)co, (float)s);
}
// (cos, sin) at a real coordinate (a block centre may be a half-integer):
// angle c * base^(-2p/(D/3)) in double, cos and sin in double, rounded to fp32.
__device__ __forceinline__ float2 rope_cs_real(float base, int D, double c, int p) {
  double theta = pow((double)base, -2.0 * (double)p / (double)(D / 3));
  double s, co;
  sincos(c * theta, &s, &co);
  return make_float2((float)co, (float)s);
}
// Rotate the channel pair (x0, x1) by (cos, sin).
__device__ __forceinline__ void rotate(float &x0, float &x1, float2 cs) {
  float y0 = x0 * cs.x - x1 * cs.y;
  float y1 = x0 * cs.y + x1 * cs.x;
  x0 = y0;
  x1 = y1;
}

__device__ __forceinline__ int site_of(const Geo &g, int z, int y, int x) {
  return (z * g.Y + y) * g.X + x;
}
// Status word bit set by a debug build's bounds check.
constexpr int kStatusDebugBounds = 4;
// The slot-map entry of a grid site. A debug build (PK_DEBUG_BOUNDS, made
// by build.py --debug) checks every such read: a site outside the grid sets
// kStatusDebugBounds in the geometry buffer's status word (which sits
// g.slot_off bytes before the map) and reads -1, so an indexing mistake
// surfaces as a status error on the host rather than as a stray read.
__device__ __forceinline__ int32_t slot_get(const Geo &g, const int32_t *slot, int64_t site) {
#ifdef PK_DEBUG_BOUNDS
  if (site < 0 || site >= (int64_t)g.Z * g.Y * g.X) {
    int *status = reinterpret_cast<int *>(const_cast<char *>(
        reinterpret_cast<const char *>(slot) - g.slot_off));
    atomicOr(status, kStatusDebugBounds);
    return -1;
  }
#endif
  return slot[site];
}
// Whether the token at memory position i, with coordinate (z, y, x), takes
// part: its coordinate is on the grid and its site's slot names it (a
// repeated coordinate leaves every token but the lowest index out).
__device__ __forceinline__ bool takes_part(const Geo &g, const int32_t *slot, int i, int z, int y,
                                           int x) {
  if (z < 0 || y < 0 || x < 0 || z >= g.Z || y >= g.Y || x >= g.X) return false;
  return slot_get(g, slot, site_of(g, z, y, x)) == i;
}
__device__ __forceinline__ int block_of(const Geo &g, int z, int y, int x) {
  return ((z / g.bz) * g.My + (y / g.by)) * g.Mx + (x / g.bx);
}
// Whether summary m is withheld from a query at (z,y,x).
__device__ __forceinline__ bool summary_excluded(const Geo &g, int z, int y, int x, int m) {
  if (g.excl == PACK3D_EXCL_NONE) return false;
  if (g.excl == PACK3D_EXCL_OWN_BLOCK) return m == block_of(g, z, y, x);
  int mz = m / (g.My * g.Mx), my = (m / g.Mx) % g.My, mx = m % g.Mx;
  int lz = max(z - 1, 0) / g.bz, hz = min(z + 1, g.Z - 1) / g.bz;
  int ly = max(y - 1, 0) / g.by, hy = min(y + 1, g.Y - 1) / g.by;
  int lx = max(x - 1, 0) / g.bx, hx = min(x + 1, g.X - 1) / g.bx;
  return mz >= lz && mz <= hz && my >= ly && my <= hy && mx >= lx && mx <= hx;
}

}  // namespace pk
