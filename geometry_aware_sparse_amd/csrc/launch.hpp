// Host-side launchers of the PACK3D kernels (one per kernel family); each
// returns the hipError_t of its launch. Shapes are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace pk {

hipError_t launch_index(const Geo &g, const int32_t *coords, void *geom, int32_t *nbr,
                        int32_t *blk, int32_t *rank, hipStream_t s);
// Zeroes the rows of tokens that take no part in up to four [B, N, len[k]]
// tensors of es-byte elements (null entries skipped).
hipError_t launch_zero_absent(const Geo &g, int es, const void *geom, const int32_t *coords,
                              void *const *rows, const int *len, hipStream_t s);
hipError_t launch_rope(const Geo &g, int dtype, const int32_t *coords, const void *x, void *y,
                       hipStream_t s);
hipError_t launch_summarize(const Geo &g, int dtype, const void *geom, const void *k,
                            const void *v, void *ks, void *vs, hipStream_t s);
// gate / oglob may be null (plain local output); when set the kernel writes
// (1-g)*O_local + g*O_global. oglob may equal out.
// bf16, D = 48: the local branch with its value sums on the matrix cores
hipError_t launch_local_tr48(const Geo &g, const void *geom, const void *q, const void *k,
                             const void *v, const void *gate, const void *og, void *out,
                             hipStream_t s);
hipError_t launch_local(const Geo &g, int dtype, const void *geom, const void *q, const void *k,
                        const void *v, const void *gate, const void *oglob, void *out,
                        hipStream_t s, bool *supported);
// lse may be null; when set it receives each (token, head)'s log-sum-exp of
// the scaled scores in log2 units ([B, N, H] fp32; -inf when nothing is
// attendable), which the backward uses to rebuild the probabilities.
hipError_t launch_global(const Geo &g, int dtype, const void *geom, const int32_t *coords,
                         const void *q, const void *ks, const void *vs, void *out, float *lse,
                         hipStream_t s, bool *supported);

// Operands of the backward (device pointers). Inputs as in the forward plus
// dout, the saved O_glob and lse_g, the recomputed summaries ks / vs and the
// fp32 intermediates; outputs dq, dk, dv, dgate in the input dtype.
struct BwdArgs {
  const void *geom;
  const int32_t *coords;
  const void *q, *k, *v, *gate, *dout, *oglob;
  const float *lse_g;
  const void *ks, *vs;
  float *qr, *dog, *delta_g, *dqg, *dks, *dvs, *lse_l, *delta_l;  // workspace
  void *dq, *dk, *dv, *dgate;
  void *const *events;  // null, or stage events: [3] after the global branch, [4] before local
  const struct BwdMfmaArgs *mfma;  // null: vector-unit global branch
};
// Matrix-core global branch of the backward (bf16, D in {48, 96}, no
// exclusion): the prepared query operands (Np = 256*ceil(N/256) grid sites),
// the relaid summaries and the split partial sums.
struct BwdMfmaArgs {
  bf16 *qn, *qt, *dn, *dt;  // [B*H, Np, D] blocked / transposed
  float *lse_p, *dl_p;      // [B*H, Np]
  int32_t *tok;             // [B, Np]
  bf16 *vk, *kt;            // [B*Hkv, Mp, D] relaid summaries
  float *dks_part, *dvs_part;  // [nsplit, B*Hkv, M, D]
  int nsplit;
};
bool bwd_global_mfma_supported(const Geo &g, int dtype);
hipError_t launch_bwd_global_mfma(const Geo &g, const BwdArgs &a, const BwdMfmaArgs &m,
                                  hipStream_t s);
// Local branch of the backward, bf16 with D in {48, 96}: D/24 lanes per site.
bool bwd_local_pair_supported(const Geo &g, int dtype);
hipError_t launch_bwd_local_pair(const Geo &g, const BwdArgs &a, hipStream_t s);
hipError_t launch_backward(const Geo &g, int dtype, const BwdArgs &a, hipStream_t s,
                           bool *supported);
hipError_t launch_mix(const Geo &g, int dtype, const void *gate, const void *ol, const void *og,
                      void *o, hipStream_t s);

// Work-item index of this workgroup such that consecutive work items land on
// the same XCD: the hardware deals workgroups round-robin over the 8 XCDs, so
// XCD x receives every 8th workgroup; give it one contiguous range instead.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  const int NX = 8;
  int x = wg % NX, idx = wg / NX;
  int base = x * (nwg / NX) + min(x, nwg % NX);
  return base + idx;
}

// (batch, head, box) of the local kernels' work item w, over nh heads: heads
// innermost (the heads of one token are adjacent in memory, so the workgroups
// of one box share cache lines), then the boxes in cubes of S x S x S boxes
// (the last cube of each axis may be cut short). Within a cube z varies
// fastest, then y, then x: a box shares more halo with its z and y
// neighbours than with its x neighbours (the boxes are longest along x), so
// those follow it closely, while its lines are still in L2. With the
// XCD-contiguous dealing above, one XCD holds a cube rather than a thin
// slab, so less of a box's halo belongs to boxes on other XCDs.
struct BoxWork {
  int b, h, tz, ty, tx;
};
__device__ __forceinline__ BoxWork box_work(int w, int nh, int ntz, int nty, int ntx) {
  const int h = w % nh;
  w /= nh;
  const int ntiles = ntz * nty * ntx;
  const int b = w / ntiles;
  int r = w - b * ntiles;
  constexpr int S = 4;  // cube edge, in boxes
  const int bz = r / (S * nty * ntx);  // slab of cubes; those before it are whole
  r -= bz * S * nty * ntx;
  const int nz = min(S, ntz - bz * S);
  const int by = r / (nz * S * ntx);   // row of cubes within the slab
  r -= by * nz * S * ntx;
  const int ny = min(S, nty - by * S);
  const int bx = r / (nz * ny * S);    // cube within the row
  r -= bx * nz * ny * S;
  const int nx = min(S, ntx - bx * S);
  return {b, h, bz * S + r % nz, by * S + (r / nz) % ny, bx * S + r / (nz * ny)};
}

}  // namespace pk
