// C ABI of the PACK3D forward (declarations and contracts in pack3d.h).
// Host-side argument validation, workspace layout and kernel launches.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <string.h>

#include "launch.hpp"

using namespace pk;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t elem_size(int dtype) { return dtype == PACK3D_BF16 ? 2 : 4; }

// Validates a descriptor and derives the kernel geometry.
int make_geo(const pack3d_desc *d, Geo *g) {
  if (!d) return PACK3D_ERR_INVALID_ARG;
  if (d->B <= 0 || d->N <= 0 || d->H <= 0 || d->D <= 0) return PACK3D_ERR_INVALID_ARG;
  if (d->dtype != PACK3D_F32 && d->dtype != PACK3D_BF16) return PACK3D_ERR_INVALID_ARG;
  if (d->exclusion < PACK3D_EXCL_NONE || d->exclusion > PACK3D_EXCL_NEIGHBOURHOOD_BLOCKS)
    return PACK3D_ERR_INVALID_ARG;
  if (!(d->rope_base > 0.0f) || !isfinite(d->rope_base)) return PACK3D_ERR_INVALID_ARG;
  if (!isfinite(d->scale)) return PACK3D_ERR_INVALID_ARG;
  if (d->flags & ~(PACK3D_VALIDATE | PACK3D_EXACT_SOFTMAX | PACK3D_SUMMARY_CENTRE))
    return PACK3D_ERR_INVALID_ARG;
  if (d->kv_heads < 0) return PACK3D_ERR_INVALID_ARG;
  const int hkv = d->kv_heads > 0 ? d->kv_heads : d->H;
  if (d->H % hkv != 0) return PACK3D_ERR_SHAPE;
  for (int a = 0; a < 3; a++)
    if (d->grid[a] <= 0 || d->block[a] <= 0) return PACK3D_ERR_SHAPE;
  if (d->D % 6 != 0) return PACK3D_ERR_SHAPE;
  const int64_t sites = (int64_t)d->grid[0] * d->grid[1] * d->grid[2];
  if (sites != d->N) return PACK3D_ERR_SHAPE;
  // element offsets are int64 in every kernel; keep token / site / summary
  // counts and per-row sizes inside int32
  if ((int64_t)d->B * d->N * d->H > ((int64_t)1 << 40)) return PACK3D_ERR_SHAPE;
  if ((int64_t)d->N * 27 > INT32_MAX || (int64_t)d->H * d->D > 1024) return PACK3D_ERR_SHAPE;
  memset(g, 0, sizeof(*g));
  g->B = d->B;
  g->N = d->N;
  g->H = d->H;
  g->D = d->D;
  g->Hkv = hkv;
  g->G = d->H / hkv;
  g->Z = d->grid[0];
  g->Y = d->grid[1];
  g->X = d->grid[2];
  g->bz = d->block[0];
  g->by = d->block[1];
  g->bx = d->block[2];
  g->Mz = (g->Z + g->bz - 1) / g->bz;
  g->My = (g->Y + g->by - 1) / g->by;
  g->Mx = (g->X + g->bx - 1) / g->bx;
  const int64_t M = (int64_t)g->Mz * g->My * g->Mx;
  const int64_t vol = (int64_t)g->bz * g->by * g->bx;
  if (M > INT32_MAX / 2 || vol > INT32_MAX / 2) return PACK3D_ERR_SHAPE;
  g->M = (int)M;
  g->vol = (int)vol;
  g->P = d->D / 6;
  g->scale = d->scale > 0.0f ? d->scale : (float)(1.0 / sqrt((double)d->D));
  g->rope_base = d->rope_base;
  g->excl = d->exclusion;
  g->flags = d->flags;
  g->slot_off = (int64_t)kAlign;
  g->table_off = (int64_t)align_up(kAlign + (size_t)sites * 4);
  return PACK3D_OK;
}

size_t geometry_bytes(const Geo &g) {
  return align_up((size_t)g.table_off + (size_t)(g.Z + g.Y + g.X + 1) * g.P * 8);
}

// k_sum [B, Hkv, Mp/32, Dp/8, 32, 8] and v_sum [B, Hkv, Mp/8, D, 8],
// Mp = 32*ceil(M/32), Dp = 8*ceil(D/8)
size_t ksum_bytes(const Geo &g, int dtype) {
  return align_up((size_t)g.B * g.Hkv * ((g.M + 31) / 32 * 32) * ((g.D + 7) / 8 * 8) *
                  elem_size(dtype));
}
size_t vsum_bytes(const Geo &g, int dtype) {
  return align_up((size_t)g.B * g.Hkv * ((g.M + 31) / 32 * 32) * g.D * elem_size(dtype));
}

int hip_status(hipError_t e) { return e == hipSuccess ? PACK3D_OK : PACK3D_ERR_HIP; }

// Synchronises and reads the status word when the caller asked for it.
int validate_coords(const pack3d_desc *d, const void *geom, hipStream_t s) {
  if (!(d->flags & PACK3D_VALIDATE)) return PACK3D_OK;
  int32_t status = 0;
  if (hipMemcpyAsync(&status, geom, sizeof(status), hipMemcpyDeviceToHost, s) != hipSuccess)
    return PACK3D_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PACK3D_ERR_HIP;
  if (status & kStatusDebugBounds) return PACK3D_ERR_INTERNAL;
  return status ? PACK3D_ERR_COORDS : PACK3D_OK;
}

// Debug builds (PK_DEBUG_BOUNDS) check the status word again once a call's
// kernels have run, under PACK3D_VALIDATE, so that a slot-map read out of
// range in any of them is reported; other builds skip it.
int debug_check(const pack3d_desc *d, const void *geom, hipStream_t s) {
#ifdef PK_DEBUG_BOUNDS
  return validate_coords(d, geom, s);
#else
  (void)d, (void)geom, (void)s;
  return PACK3D_OK;
#endif
}

}  // namespace

extern "C" {

int pack3d_abi_version(void) { return PACK3D_ABI_VERSION; }

const char *pack3d_strerror(int status) {
  switch (status) {
    case PACK3D_OK: return "success";
    case PACK3D_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size or bad enum)";
    case PACK3D_ERR_SHAPE: return "invalid shape (N != Z*Y*X, D not a multiple of 6, block < 1, H not a multiple of kv_heads, or size limits)";
    case PACK3D_ERR_WORKSPACE: return "workspace too small";
    case PACK3D_ERR_UNSUPPORTED: return "dtype / head-dim / exclusion combination not built";
    case PACK3D_ERR_HIP: return "HIP runtime or launch failure";
    case PACK3D_ERR_COORDS: return "coordinate off the grid or duplicated";
    case PACK3D_ERR_INTERNAL: return "a debug build's bounds check found a slot-map read out of range";
    default: return "unknown pack3d status";
  }
}

int64_t pack3d_num_summaries(const pack3d_desc *desc) {
  Geo g;
  int rc = make_geo(desc, &g);
  return rc ? rc : (int64_t)g.M;
}

int pack3d_geometry_layout(const pack3d_desc *desc, size_t *slot_offset, size_t *table_offset,
                           size_t *bytes) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (slot_offset) *slot_offset = (size_t)g.slot_off;
  if (table_offset) *table_offset = (size_t)g.table_off;
  if (bytes) *bytes = geometry_bytes(g);
  return PACK3D_OK;
}

int pack3d_geometry_bytes(const pack3d_desc *desc, size_t *bytes) {
  if (!bytes) return PACK3D_ERR_INVALID_ARG;
  return pack3d_geometry_layout(desc, nullptr, nullptr, bytes);
}

int pack3d_workspace_bytes(const pack3d_desc *desc, size_t *bytes) {
  Geo g;
  if (!bytes) return PACK3D_ERR_INVALID_ARG;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  *bytes = geometry_bytes(g) + ksum_bytes(g, desc->dtype) + vsum_bytes(g, desc->dtype);
  return PACK3D_OK;
}

int pack3d_index_build(const pack3d_desc *desc, const int32_t *coords, void *geom,
                       int32_t *nbr_out, int32_t *block_out, int32_t *rank_out, void *stream) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (!coords || !geom) return PACK3D_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = hip_status(launch_index(g, coords, geom, nbr_out, block_out, rank_out, s));
  if (rc) return rc;
  return validate_coords(desc, geom, s);
}

int pack3d_rope_coords(const pack3d_desc *desc, const int32_t *coords, const void *x,
                       void *x_rot, void *stream) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (!coords || !x || !x_rot) return PACK3D_ERR_INVALID_ARG;
  return hip_status(launch_rope(g, desc->dtype, coords, x, x_rot, static_cast<hipStream_t>(stream)));
}

int pack3d_block_summarize(const pack3d_desc *desc, const void *geom, const void *k,
                           const void *v, void *k_sum, void *v_sum, void *stream) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (!geom || !k || !v || !k_sum || !v_sum) return PACK3D_ERR_INVALID_ARG;
  if ((rc = hip_status(launch_summarize(g, desc->dtype, geom, k, v, k_sum, v_sum,
                                        static_cast<hipStream_t>(stream)))))
    return rc;
  return debug_check(desc, geom, static_cast<hipStream_t>(stream));
}

int pack3d_local_attn(const pack3d_desc *desc, const void *geom, const void *q, const void *k,
                      const void *v, void *o_local, void *stream) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (!geom || !q || !k || !v || !o_local) return PACK3D_ERR_INVALID_ARG;
  bool ok = false;
  hipError_t e = launch_local(g, desc->dtype, geom, q, k, v, nullptr, nullptr, o_local,
                              static_cast<hipStream_t>(stream), &ok);
  if (!ok) return PACK3D_ERR_UNSUPPORTED;
  if ((rc = hip_status(e))) return rc;
  return debug_check(desc, geom, static_cast<hipStream_t>(stream));
}

int pack3d_global_attn(const pack3d_desc *desc, const void *geom, const int32_t *coords,
                       const void *q, const void *k_sum, const void *v_sum, void *o_global,
                       void *stream) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (!geom || !coords || !q || !k_sum || !v_sum || !o_global) return PACK3D_ERR_INVALID_ARG;
  bool ok = false;
  hipError_t e = launch_global(g, desc->dtype, geom, coords, q, k_sum, v_sum, o_global, nullptr,
                               static_cast<hipStream_t>(stream), &ok);
  if (!ok) return PACK3D_ERR_UNSUPPORTED;
  if ((rc = hip_status(e))) return rc;
  return debug_check(desc, geom, static_cast<hipStream_t>(stream));
}

int pack3d_mix(const pack3d_desc *desc, const void *gate, const void *o_local,
               const void *o_global, void *o, void *stream) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (!gate || !o_local || !o_global || !o) return PACK3D_ERR_INVALID_ARG;
  return hip_status(
      launch_mix(g, desc->dtype, gate, o_local, o_global, o, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

bool shape_supported(const pack3d_desc *desc, const Geo &g) {
  const bool mfma = desc->dtype == PACK3D_BF16 && desc->exclusion == PACK3D_EXCL_NONE &&
                    (g.D == 48 || g.D == 96);
  const bool valu = g.D == 6 || g.D == 12 || g.D == 24 || g.D == 48 || g.D == 96;
  return mfma || valu;
}

// saved = [O_glob [B, N, H, D] in dtype | lse_glob [B, N, H] fp32], 256-aligned
size_t saved_oglob_bytes(const Geo &g, int dtype) {
  return align_up((size_t)g.B * g.N * g.H * g.D * elem_size(dtype));
}
size_t saved_bytes(const Geo &g, int dtype) {
  return saved_oglob_bytes(g, dtype) + align_up((size_t)g.B * g.N * g.H * 4);
}

// The forward pipeline; oglob / lse are where the global branch writes (o
// itself and no lse for inference, the saved buffer for training).
int forward_impl(const pack3d_desc *desc, const int32_t *coords, const void *q, const void *k,
                 const void *v, const void *gate, void *o, void *oglob, float *lse, void *ws,
                 size_t ws_bytes, void *stream, void *const *stage_events) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (!coords || !q || !k || !v || !gate || !o || !ws) return PACK3D_ERR_INVALID_ARG;
  const size_t gbytes = geometry_bytes(g), kbytes = ksum_bytes(g, desc->dtype),
               vbytes = vsum_bytes(g, desc->dtype);
  if (ws_bytes < gbytes + kbytes + vbytes) return PACK3D_ERR_WORKSPACE;
  // shape support is decided before anything is enqueued
  if (!shape_supported(desc, g)) return PACK3D_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *base = static_cast<char *>(ws);
  void *geom = base;
  void *ksum = base + gbytes;
  void *vsum = base + gbytes + kbytes;
  auto mark = [&](int idx) -> int {
    if (!stage_events || !stage_events[idx]) return PACK3D_OK;  // NULL entries are skipped
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(stage_events[idx]), s));
  };
  bool ok = true;
  if ((rc = mark(0))) return rc;
  if ((rc = hip_status(launch_index(g, coords, geom, nullptr, nullptr, nullptr, s)))) return rc;
  if ((rc = mark(1))) return rc;
  if ((rc = validate_coords(desc, geom, s))) return rc;
  if ((rc = mark(2))) return rc;
  if ((rc = hip_status(launch_summarize(g, desc->dtype, geom, k, v, ksum, vsum, s)))) return rc;
  if ((rc = mark(3))) return rc;
  if ((rc = mark(4))) return rc;
  if ((rc = hip_status(launch_global(g, desc->dtype, geom, coords, q, ksum, vsum, oglob, lse, s, &ok))))
    return rc;
  if (!ok) return PACK3D_ERR_UNSUPPORTED;
  if ((rc = mark(5))) return rc;
  if ((rc = mark(6))) return rc;
  if ((rc = hip_status(launch_local(g, desc->dtype, geom, q, k, v, gate, oglob, o, s, &ok)))) return rc;
  if (!ok) return PACK3D_ERR_UNSUPPORTED;
  if (oglob != o) {
    // training: the global branch wrote into the saved buffer, so the rows of
    // o that the local kernel does not reach (tokens taking no part) are
    // zeroed here, as the global kernel zeroes them in the inference forward
    void *rows[4] = {o, nullptr, nullptr, nullptr};
    const int len[4] = {g.H * g.D, 0, 0, 0};
    if ((rc = hip_status(launch_zero_absent(g, (int)elem_size(desc->dtype), geom, coords, rows,
                                            len, s))))
      return rc;
  }
  if ((rc = mark(7))) return rc;
  return debug_check(desc, geom, s);
}

// Backward workspace: geometry | k_sum | v_sum | fp32 intermediates, then
// the matrix-core operands when that path runs (the vector-unit query
// buffers are left out there)
struct BwdLayout {
  size_t geom, ks, vs, qr, dog, delta_g, dqg, dks, dvs, lse_l, delta_l;
  bool mfma;
  int nsplit;
  size_t qn, qt, dn, dt, lse_p, dl_p, tok, vk, kt, dks_part, dvs_part;
  size_t total;
};
BwdLayout bwd_layout(const Geo &g, int dtype) {
  BwdLayout L;
  const size_t rows = (size_t)g.B * g.N * g.H;
  const size_t sum = (size_t)g.B * g.Hkv * g.M * g.D * 4;
  L.mfma = bwd_global_mfma_supported(g, dtype);
  size_t off = 0;
  auto take = [&](size_t n) { size_t at = off; off += align_up(n); return at; };
  L.geom = take(geometry_bytes(g));
  L.ks = take(ksum_bytes(g, dtype));
  L.vs = take(vsum_bytes(g, dtype));
  L.qr = take(L.mfma ? 0 : rows * g.D * 4);
  L.dog = take(L.mfma ? 0 : rows * g.D * 4);
  L.delta_g = take(L.mfma ? 0 : rows * 4);
  L.dqg = take(rows * g.D * 4);
  L.dks = take(sum);
  L.dvs = take(sum);
  L.lse_l = take(rows * 4);
  L.delta_l = take(rows * 4);
  L.nsplit = 1;
  L.qn = L.qt = L.dn = L.dt = L.lse_p = L.dl_p = L.tok = L.vk = L.kt = L.dks_part =
      L.dvs_part = 0;
  if (L.mfma) {
    // the summary side runs (Mp/128) x B x Hkv workgroups of 4 waves per
    // split: split the query sites until about 2048 workgroups fill the chip
    const size_t Np = ((size_t)g.N + 255) / 256 * 256, Mp = ((size_t)g.M + 31) / 32 * 32;
    const size_t wgs = (Mp / 32 + 3) / 4 * g.B * g.Hkv;
    L.nsplit = (int)std::min<size_t>(16, std::max<size_t>(1, (2048 + wgs - 1) / wgs));
    const size_t prow = (size_t)g.B * g.H * Np;
    L.qn = take(prow * g.D * 2);
    L.qt = take(prow * g.D * 2);
    L.dn = take(prow * g.D * 2);
    L.dt = take(prow * g.D * 2);
    L.lse_p = take(prow * 4);
    L.dl_p = take(prow * 4);
    L.tok = take((size_t)g.B * Np * 4);
    L.vk = take((size_t)g.B * g.Hkv * Mp * g.D * 2);
    L.kt = take((size_t)g.B * g.Hkv * Mp * g.D * 2);
    L.dks_part = take(sum * L.nsplit);
    L.dvs_part = take(sum * L.nsplit);
  }
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

int pack3d_forward(const pack3d_desc *desc, const int32_t *coords, const void *q, const void *k,
                   const void *v, const void *gate, void *o, void *ws, size_t ws_bytes,
                   void *stream, void *const *stage_events) {
  return forward_impl(desc, coords, q, k, v, gate, o, o, nullptr, ws, ws_bytes, stream,
                      stage_events);
}

}  // extern "C"

// Scratch of pack3d_forward_noalloc: the forward's workspace (geometry
// metadata, k_sum, v_sum) in a device array of fixed size, one copy per GPU,
// held until the process ends. In host code `scratch` names a host-side
// stand-in, never the device memory: its address on a device is taken once
// per device with hipGetSymbolAddress (that device current) and only that
// address is handed to kernels.
static __device__ __align__(256) char scratch[PACK3D_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void *scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the
// first call there.
int device_scratch(hipStream_t s, void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PACK3D_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PACK3D_ERR_UNSUPPORTED;
  if (s) {  // the stream must belong to the current device
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return PACK3D_ERR_HIP;
    if (sdev != dev) return PACK3D_ERR_INVALID_ARG;
  }
  std::call_once(scratch_once[dev], [dev] {
    void *p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev]) return PACK3D_ERR_HIP;
  *ptr = scratch_ptr[dev];
  return PACK3D_OK;
}

}  // namespace

extern "C" {

int pack3d_forward_noalloc(const pack3d_desc *desc, const int32_t *coords, const void *q,
                           const void *k, const void *v, const void *gate, void *o,
                           void *stream) {
  size_t need = 0;
  int rc = pack3d_workspace_bytes(desc, &need);
  if (rc) return rc;
  if (need > (size_t)PACK3D_NOALLOC_SCRATCH_BYTES) return PACK3D_ERR_WORKSPACE;
  if (!coords || !q || !k || !v || !gate || !o) return PACK3D_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void *ws = nullptr;
  if ((rc = device_scratch(s, &ws))) return rc;
  // every byte the forward reads from its workspace is written by it first
  // (status word, slot map, RoPE table, summaries with their padding), so
  // nothing left by an earlier call needs clearing
  return forward_impl(desc, coords, q, k, v, gate, o, o, nullptr, ws,
                      (size_t)PACK3D_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int pack3d_saved_bytes(const pack3d_desc *desc, size_t *bytes) {
  Geo g;
  if (!bytes) return PACK3D_ERR_INVALID_ARG;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  *bytes = saved_bytes(g, desc->dtype);
  return PACK3D_OK;
}

int pack3d_forward_train(const pack3d_desc *desc, const int32_t *coords, const void *q,
                         const void *k, const void *v, const void *gate, void *o, void *saved,
                         size_t saved_bytes_, void *ws, size_t ws_bytes, void *stream,
                         void *const *stage_events) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (!saved) return PACK3D_ERR_INVALID_ARG;
  if (saved_bytes_ < saved_bytes(g, desc->dtype)) return PACK3D_ERR_WORKSPACE;
  char *sv = static_cast<char *>(saved);
  return forward_impl(desc, coords, q, k, v, gate, o, sv,
                      reinterpret_cast<float *>(sv + saved_oglob_bytes(g, desc->dtype)), ws,
                      ws_bytes, stream, stage_events);
}

int pack3d_backward_workspace_bytes(const pack3d_desc *desc, size_t *bytes) {
  Geo g;
  if (!bytes) return PACK3D_ERR_INVALID_ARG;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  *bytes = bwd_layout(g, desc->dtype).total;
  return PACK3D_OK;
}

int pack3d_backward(const pack3d_desc *desc, const int32_t *coords, const void *q, const void *k,
                    const void *v, const void *gate, const void *saved, size_t saved_bytes_,
                    const void *dout, void *dq, void *dk, void *dv, void *dgate, void *ws,
                    size_t ws_bytes, void *stream, void *const *stage_events) {
  Geo g;
  int rc = make_geo(desc, &g);
  if (rc) return rc;
  if (!coords || !q || !k || !v || !gate || !saved || !dout || !dq || !dk || !dv || !dgate || !ws)
    return PACK3D_ERR_INVALID_ARG;
  if (saved_bytes_ < saved_bytes(g, desc->dtype)) return PACK3D_ERR_WORKSPACE;
  const BwdLayout L = bwd_layout(g, desc->dtype);
  if (ws_bytes < L.total) return PACK3D_ERR_WORKSPACE;
  if (!shape_supported(desc, g)) return PACK3D_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *base = static_cast<char *>(ws);
  auto mark = [&](int idx) -> int {
    if (!stage_events || !stage_events[idx]) return PACK3D_OK;  // NULL entries are skipped
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(stage_events[idx]), s));
  };
  BwdArgs a;
  a.geom = base + L.geom;
  a.coords = coords;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate = gate;
  a.dout = dout;
  a.oglob = saved;
  a.lse_g = reinterpret_cast<const float *>(static_cast<const char *>(saved) +
                                            saved_oglob_bytes(g, desc->dtype));
  a.ks = base + L.ks;
  a.vs = base + L.vs;
  a.qr = reinterpret_cast<float *>(base + L.qr);
  a.dog = reinterpret_cast<float *>(base + L.dog);
  a.delta_g = reinterpret_cast<float *>(base + L.delta_g);
  a.dqg = reinterpret_cast<float *>(base + L.dqg);
  a.dks = reinterpret_cast<float *>(base + L.dks);
  a.dvs = reinterpret_cast<float *>(base + L.dvs);
  a.lse_l = reinterpret_cast<float *>(base + L.lse_l);
  a.delta_l = reinterpret_cast<float *>(base + L.delta_l);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dgate = dgate;
  a.events = stage_events;
  BwdMfmaArgs mf;
  a.mfma = nullptr;
  if (L.mfma) {
    mf.qn = reinterpret_cast<bf16 *>(base + L.qn);
    mf.qt = reinterpret_cast<bf16 *>(base + L.qt);
    mf.dn = reinterpret_cast<bf16 *>(base + L.dn);
    mf.dt = reinterpret_cast<bf16 *>(base + L.dt);
    mf.lse_p = reinterpret_cast<float *>(base + L.lse_p);
    mf.dl_p = reinterpret_cast<float *>(base + L.dl_p);
    mf.tok = reinterpret_cast<int32_t *>(base + L.tok);
    mf.vk = reinterpret_cast<bf16 *>(base + L.vk);
    mf.kt = reinterpret_cast<bf16 *>(base + L.kt);
    mf.dks_part = reinterpret_cast<float *>(base + L.dks_part);
    mf.dvs_part = reinterpret_cast<float *>(base + L.dvs_part);
    mf.nsplit = L.nsplit;
    a.mfma = &mf;
  }
  if ((rc = mark(0))) return rc;
  if ((rc = hip_status(launch_index(g, coords, base + L.geom, nullptr, nullptr, nullptr, s))))
    return rc;
  if ((rc = validate_coords(desc, base + L.geom, s))) return rc;
  if ((rc = hip_status(launch_summarize(g, desc->dtype, base + L.geom, k, v, base + L.ks,
                                        base + L.vs, s))))
    return rc;
  if ((rc = mark(1))) return rc;
  if ((rc = mark(2))) return rc;
  bool ok = true;
  if ((rc = hip_status(launch_backward(g, desc->dtype, a, s, &ok)))) return rc;
  if (!ok) return PACK3D_ERR_UNSUPPORTED;
  if ((rc = mark(5))) return rc;
  return debug_check(desc, base + L.geom, s);
}

}  // extern "C"
