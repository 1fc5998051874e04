/*
 * pack3d.h -- C ABI of PACK3D local-global attention on gfx950: the forward
 * pass, its stages one by one, and the backward pass.
 *
 * The operator (Geometry Matters in Packed 3D Attention; "project page" =
 * the Pack3D site, "paper summary" = the arXiv 2610.38694 abstract page):
 * tokens of a 3D grid are stored in any memory order (raster, Morton,
 * block-contiguous, random) and each carries its integer grid coordinate
 * (project page Ch. 1; paper summary §3.1, §B.1). Queries and keys are
 * rotated with axial RoPE at those coordinates, never at the memory index
 * (project page Ch. 3, Contract 3). Each query attends exactly to its 3x3x3
 * coordinate neighbourhood (Contract 1) and to every block summary, built by
 * rotating keys first and mean-pooling them per contiguous 3D block
 * (Contract 2 and "Rotate first, then pool"; paper summary §3.2, §B.5). A
 * tokenwise gate mixes the two branches (paper summary §3.3). The operator is
 * trained end to end (paper summary §1, §3.4): pack3d_forward_train and
 * pack3d_backward give the gradients with respect to q, k, v and the gate.
 *
 * Conventions shared by every entry point
 *  - Pointers named q, k, v, gate, o, x, k_sum, v_sum, geom, coords, ws and
 *    the *_out arrays are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains device memory (pack3d_forward_noalloc
 *    uses a fixed device array inside the library instead of a workspace).
 *  - Layouts (row-major, C order), with Hkv = desc->kv_heads (H when 0):
 *      q, o, o_local, o_global, x       : [B, N, H, D] in packed memory order
 *      k, v                             : [B, N, Hkv, D], same packing
 *      gate                             : [B, N, H] (gate logits G)
 *      coords                           : int32 [N, 3] = (z, y, x) of the
 *                                         token stored at each position; one
 *                                         packing shared by the whole batch
 *      k_sum, v_sum                     : summaries of blocks in block-id
 *                                         order m = (mz*My + my)*Mx + mx,
 *                                         blocked for the matrix-core kernel,
 *                                         with M padded to Mp = 32*ceil(M/32)
 *                                         (padding slots are zero):
 *        k_sum [B, Hkv, Mp/32, Dp/8, 32, 8]: key summary (m, d) of KV
 *                                         head h at [b, h, m/32, d/8, m%32,
 *                                         d%8], with D padded to
 *                                         Dp = 8*ceil(D/8) (zero)
 *        v_sum [B, Hkv, Mp/8, D, 8]     : value summary (m, d) at
 *                                         [b, h, m/8, d, m%8]
 *  - Grouped key/value heads (GQA, MQA): keys, values and the summaries
 *    exist per KV head (project page Ch. 3, Contract 2 counts summaries per
 *    KV head; paper summary §D.1 shares work within KV groups). Query head h
 *    reads KV head h / (H / Hkv): consecutive query heads form a group.
 *    Hkv == H is multi-head attention, Hkv == 1 multi-query attention.
 *    Element type of q/k/v/gate/o/x/k_sum/v_sum is desc->dtype.
 *  - stream is a hipStream_t passed as void* (NULL = default stream). Every
 *    call only enqueues work on it and returns; results are ready when the
 *    stream reaches that point. Calls are reentrant: the library keeps no
 *    mutable global state, except pack3d_forward_noalloc's per-GPU array.
 *  - Return value: PACK3D_OK or a negative pack3d_status. Argument checks run
 *    on the host before anything is enqueued; nothing is launched when they
 *    fail. Coordinate errors are detected on the device: kernels never read
 *    out of bounds, and the error is reported to the host only when
 *    desc->flags has PACK3D_VALIDATE (the call then synchronises the stream).
 *  - Debug build (lib/libpack3d_debug.so, built by build.py --debug): every
 *    slot-map read in every kernel is checked against the grid; one out of
 *    range sets bit 2 of the status word and reads as an empty site. Under
 *    PACK3D_VALIDATE, the entry points that run kernels reading the map
 *    then synchronise once more at their end and return PACK3D_ERR_INTERNAL
 *    if the bit is set. Results are otherwise those of the normal build.
 *  - Without PACK3D_VALIDATE a bad coordinate is resolved deterministically.
 *    A token whose coordinate is off the grid takes no part. A site claimed
 *    by several tokens goes to the lowest memory index among them, and the
 *    others take no part. A token that takes no part is nobody's neighbour
 *    and no block's member; its output row from pack3d_global_attn,
 *    pack3d_forward and pack3d_forward_train is zero, its saved log-sum-exp
 *    is -inf, and its dq, dk, dv and dgate rows from pack3d_backward are
 *    zero. pack3d_local_attn visits grid sites only, so it leaves that row of
 *    o_local unwritten. A grid site with no token is skipped by every
 *    kernel.
 *
 * Readings taken where the pages are silent (their formulas did not survive):
 * RoPE channels are three contiguous chunks of D/3 for z, y, x; plane p of a
 * chunk is the channel pair (2p, 2p+1) turned by c_axis * base^(-2p/(D/3));
 * the neighbourhood is Chebyshev radius 1 including the query, clipped at the
 * grid edge; the softmax scale defaults to 1/sqrt(D) in both branches;
 * summaries are arithmetic means over the members present (blocks tile the
 * grid from coordinate 0; edge blocks may be partial); every query attends to
 * all M summaries by default; the gate is g = sigmoid(G) per token and head
 * and O = (1-g)*O_local + g*O_global.
 */
#ifndef PACK3D_H
#define PACK3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PACK3D_ABI_VERSION 2

typedef enum pack3d_status {
  PACK3D_OK = 0,
  PACK3D_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad enum */
  PACK3D_ERR_SHAPE = -2,       /* N != Z*Y*X, D % 6, block < 1, H % kv_heads, overflow */
  PACK3D_ERR_WORKSPACE = -3,   /* workspace or saved buffer smaller than required  */
  PACK3D_ERR_UNSUPPORTED = -4, /* dtype / D / exclusion combination not built */
  PACK3D_ERR_HIP = -5,         /* a HIP launch or runtime call failed */
  PACK3D_ERR_COORDS = -6,      /* coordinate off the grid or duplicated (VALIDATE only) */
  PACK3D_ERR_INTERNAL = -7     /* debug builds only: a slot-map read out of range (VALIDATE) */
} pack3d_status;

typedef enum pack3d_dtype { PACK3D_F32 = 0, PACK3D_BF16 = 1 } pack3d_dtype;

/* Which summaries a query may not attend to. The pages say both that the
 * summaries carry only the nonlocal context (paper summary §3.2) and that
 * every query attends to all of them (project page Ch. 3, Contract 2; the
 * N^2/v interaction count of paper summary §B.10); NONE follows the latter. */
typedef enum pack3d_exclusion {
  PACK3D_EXCL_NONE = 0,                /* attend to all M summaries (default) */
  PACK3D_EXCL_OWN_BLOCK = 1,           /* skip the block holding the query */
  PACK3D_EXCL_NEIGHBOURHOOD_BLOCKS = 2 /* skip every block meeting the clipped 3x3x3 */
} pack3d_exclusion;

#define PACK3D_VALIDATE 0x1u /* synchronise and report coordinate errors */
/* Global branch on matrix cores: by default scores go through exp2 without a
 * running maximum (exact up to rounding while every score is below 2^7 in
 * log2 units) and any query whose softmax denominator leaves the safe range
 * is redone by an exact two-pass softmax. This flag sends every query
 * through the two-pass softmax (maximum first, then the sums). */
#define PACK3D_EXACT_SOFTMAX 0x2u
/* Summary-centre variant of the compressed branch (paper summary §B.7, §B.8;
 * project page Ch. 3): the key summary is the mean of the UNROTATED member
 * keys, rotated once at the block centre (origin + (extent - 1) / 2 along
 * each axis, the extent clipped at the grid edge; a half-integer coordinate
 * for an even extent). Without it every key is rotated at its own coordinate
 * before pooling, which keeps each member's displacement from the query
 * exactly (the default). Values are pooled the same way in both. */
#define PACK3D_SUMMARY_CENTRE 0x4u

typedef struct pack3d_desc {
  int32_t B, N, H, D;  /* batch, tokens, heads, head dim (D % 6 == 0)         */
  int32_t grid[3];     /* Z, Y, X; every grid site holds one token: N == Z*Y*X */
  int32_t block[3];    /* bz, by, bx >= 1: summary block shape                  */
  float rope_base;     /* RoPE base (10000 in the measured workloads); > 0      */
  float scale;         /* softmax scale; <= 0 selects 1/sqrt(D)                  */
  int32_t dtype;       /* pack3d_dtype of every float tensor                     */
  int32_t exclusion;   /* pack3d_exclusion                                       */
  uint32_t flags;      /* PACK3D_VALIDATE | PACK3D_EXACT_SOFTMAX | ..._CENTRE     */
  int32_t kv_heads;    /* key/value heads Hkv; 0 selects H; H % Hkv == 0         */
} pack3d_desc;

/* Library ABI version (PACK3D_ABI_VERSION). */
int pack3d_abi_version(void);

/* Human-readable text for a pack3d_status; never NULL. */
const char *pack3d_strerror(int status);

/* Number of summaries M = ceil(Z/bz)*ceil(Y/by)*ceil(X/bx) for desc, or a
 * negative pack3d_status when desc is invalid. */
int64_t pack3d_num_summaries(const pack3d_desc *desc);

/* ---------------------------------------------------------------------------
 * Geometry metadata (what a repack must carry with each token: coordinate,
 * neighbourhood edges, block membership and within-block slot; project page
 * Ch. 4, Prop. 2). It lives in one caller buffer `geom` of
 * pack3d_geometry_bytes() bytes, 256-byte aligned, laid out as:
 *   [0, 256)               int32 status word (bit 0: coordinate off the grid,
 *                          bit 1: coordinate duplicated, bit 2: a debug
 *                          build's bounds check fired); bytes [64, 128)
 *                          are zero (read in place of an absent block
 *                          member); the rest is padding
 *   [slot_offset, ...)     int32 slot map [Z*Y*X]: slot[(z*Y + y)*X + x] =
 *                          memory position of the token at (z,y,x) (the
 *                          lowest one when several claim the site), -1 if
 *                          none
 *   [table_offset, ...)    float32 RoPE table [(Z+Y+X+1) * (D/6)][2]: entry
 *                          (axis_start + c)*(D/6) + p holds (cos, sin) of
 *                          c * base^(-2p/(D/3)), evaluated in double and
 *                          rounded; axis_start is 0, Z, Z+Y for z, y, x;
 *                          the last row (Z+Y+X)*(D/6) + p holds the same at
 *                          c = 1/2 (block centres of even extent)
 * Offsets are reported by pack3d_geometry_layout. */
int pack3d_geometry_bytes(const pack3d_desc *desc, size_t *bytes);
int pack3d_geometry_layout(const pack3d_desc *desc, size_t *slot_offset, size_t *table_offset,
                           size_t *bytes);

/* Builds the geometry metadata from the coordinates: clears the status word
 * and slot map, scatters slot[site(c_i)] = i, flags off-grid or repeated
 * coordinates and fills the RoPE table. Optional outputs (device, may be
 * NULL), all int32 over memory positions i:
 *   nbr_out   [N, 27]: memory position of the neighbour at offset
 *             (k/9 - 1, (k/3)%3 - 1, k%3 - 1), -1 off the grid or empty
 *   block_out [N]: block id floor(z/bz)*My*Mx + floor(y/by)*Mx + floor(x/bx)
 *   rank_out  [N]: within-block slot ((z%bz)*by + y%by)*bx + x%bx
 * Index results are exact integers. Under PACK3D_VALIDATE returns
 * PACK3D_ERR_COORDS when the status word is non-zero. */
int pack3d_index_build(const pack3d_desc *desc, const int32_t *coords, void *geom,
                       int32_t *nbr_out, int32_t *block_out, int32_t *rank_out, void *stream);

/* Axial RoPE at grid coordinates, materialised (project page Ch. 3,
 * Contract 3; paper summary §B.2): x_rot = R(c_i) x_i for every batch, token
 * and head; x_rot may equal x (in place) but may not partially overlap it.
 * Computed in fp32 from cos/sin evaluated in double; bf16 output is rounded
 * to nearest even. The other entry points take UNROTATED q and k and rotate
 * them as they load them; this call exists for tests and for callers that
 * want rotated tensors. x has desc->H heads; to rotate keys with fewer KV
 * heads, pass a descriptor whose H is the KV head count. */
int pack3d_rope_coords(const pack3d_desc *desc, const int32_t *coords, const void *x,
                       void *x_rot, void *stream);

/* Rotate-then-pool block summaries (project page Ch. 3, "Rotate first, then
 * pool"; paper summary §3.2, §B.5): for every KV head h,
 * k_sum[b,h,m] = mean over the members j of block m of R(c_j) k[b,j,h];
 * v_sum[b,h,m] = mean of v[b,j,h]. Members are
 * summed in fp32 in within-block-slot order, so the result does not depend on
 * the packing. geom must hold metadata built by pack3d_index_build for the
 * same desc. Blocks with no member present get zeros. */
int pack3d_block_summarize(const pack3d_desc *desc, const void *geom, const void *k,
                           const void *v, void *k_sum, void *v_sum, void *stream);

/* Exact local attention (project page Ch. 3, Contract 1; paper summary §3.2,
 * §3.5): for each token i, head h, softmax over the valid tokens j of the
 * 3x3x3 coordinate neighbourhood of scale * <R(c_i) q_i, R(c_j) k_j>, then
 * the weighted sum of the unrotated v_j (k and v of KV head h / (H / Hkv)).
 * fp32 softmax and accumulation;
 * neighbours are visited in the fixed offset order. o_local may not alias
 * q, k or v. */
int pack3d_local_attn(const pack3d_desc *desc, const void *geom, const void *q, const void *k,
                      const void *v, void *o_local, void *stream);

/* Query-to-summary attention (project page Ch. 3, Contract 2; paper summary
 * §3.5, §B.10): for each token i, head h, softmax over the summaries m (all
 * of them, or those desc->exclusion leaves) of
 * scale * <R(c_i) q_i, k_sum[b,hk,m]>, then the weighted sum of
 * v_sum[b,hk,m], hk = h / (H / Hkv);
 * zero when every summary is excluded. bf16 with D in {48, 96} and no
 * exclusion runs on bf16 matrix cores with an fp32 online softmax; every
 * other case runs an fp32 vector kernel. o_global may not alias q. */
int pack3d_global_attn(const pack3d_desc *desc, const void *geom, const int32_t *coords,
                       const void *q, const void *k_sum, const void *v_sum, void *o_global,
                       void *stream);

/* Tokenwise mix (paper summary §3.3): g = 1/(1+exp(-gate[b,i,h])),
 * o = (1-g)*o_local + g*o_global, elementwise in fp32. o may alias o_local
 * or o_global exactly. */
int pack3d_mix(const pack3d_desc *desc, const void *gate, const void *o_local,
               const void *o_global, void *o, void *stream);

/* Workspace needed by pack3d_forward: the geometry metadata followed by
 * k_sum and v_sum, each 256-byte aligned. */
int pack3d_workspace_bytes(const pack3d_desc *desc, size_t *bytes);

/* The whole PACK3D operator (project page Ch. 3, Contracts 1-3 and "Rotate
 * first, then pool"; paper summary §3.2, §3.3, §3.5): for each token i and
 * head h, O = (1-g)*O_local + g*O_global with g = sigmoid(gate), where the
 * two branches are those of pack3d_local_attn and pack3d_global_attn over the
 * summaries of pack3d_block_summarize, all from UNROTATED q and k. Stream-
 * ordered: index build, summaries, global branch (written into o), then
 * local branch fused with the mix (reads o, writes o). Equivalent to the
 * staged calls above; o must not alias q, k, v or gate. ws: device workspace of at least pack3d_workspace_bytes bytes
 * (ws_bytes says how large it is). stage_events: NULL, or an array of
 * 2*PACK3D_NUM_STAGES hipEvent_t (as void*) that are recorded on stream
 * before and after each stage (index, summarize, global, local+mix), for
 * timing; a NULL entry is skipped. Each recorded event costs a few
 * microseconds of stream time, so time a stage with its own two only. */
#define PACK3D_NUM_STAGES 4
int pack3d_forward(const pack3d_desc *desc, const int32_t *coords, const void *q, const void *k,
                   const void *v, const void *gate, void *o, void *ws, size_t ws_bytes,
                   void *stream, void *const *stage_events);

/* pack3d_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operator, kernels and results (bit for bit) as pack3d_forward, but
 * the workspace is a device array inside the library of
 * PACK3D_NOALLOC_SCRATCH_BYTES bytes, one per GPU, kept until the process
 * ends; the call itself allocates nothing. It runs on the current device, and
 * stream (NULL = default stream) must belong to it (else
 * PACK3D_ERR_INVALID_ARG). Returns PACK3D_ERR_WORKSPACE, with nothing
 * launched, when pack3d_workspace_bytes(desc) exceeds the array. Every call
 * on one GPU shares that GPU's array: calls that may overlap on one GPU
 * (different streams, or host threads) race and must be serialised by the
 * caller. The first call on a device looks up the array's device address. */
#define PACK3D_NOALLOC_SCRATCH_BYTES (32u << 20)
int pack3d_forward_noalloc(const pack3d_desc *desc, const int32_t *coords, const void *q,
                           const void *k, const void *v, const void *gate, void *o,
                           void *stream);

/* ---------------------------------------------------------------------------
 * Training (paper summary §1, §3.4: the operator is trained end to end, with
 * a backward that follows the forward's streamed access pattern).
 *
 * pack3d_forward_train is pack3d_forward that also fills `saved`, a device
 * buffer of at least pack3d_saved_bytes bytes, laid out as
 *   [0, ...)          O_glob [B, N, H, D] in desc->dtype (the global branch)
 *   [256-aligned)     lse [B, N, H] fp32: log2 of the global softmax
 *                     denominator of the scores scaled by scale * log2(e)
 *                     (-inf when no summary is attendable)
 * o is the same as pack3d_forward's. saved_bytes says how large saved is.
 *
 * pack3d_backward takes the forward's inputs, its saved buffer and dout =
 * dL/dO [B, N, H, D] and writes the gradients of L with respect to the
 * UNROTATED inputs: dq [B, N, H, D], dk and dv [B, N, Hkv, D] (summed over
 * each KV head's group of query heads) and dgate [B, N, H] (with respect to
 * the gate logits G), all in desc->dtype. It recomputes the geometry, the
 * summaries and both softmaxes (the global one from the saved log-sum-exp);
 * accumulation is fp32. Every reduction has a fixed order: results are
 * deterministic, and a repack of the tokens permutes every gradient bit for
 * bit. ws: device workspace of at least pack3d_backward_workspace_bytes
 * bytes. stage_events: NULL or 2*PACK3D_NUM_BWD_STAGES hipEvent_t recorded
 * around each stage (geometry + summaries, global branch, local branch);
 * a NULL entry is skipped.
 * None of the outputs may alias an input. */
int pack3d_saved_bytes(const pack3d_desc *desc, size_t *bytes);
int pack3d_forward_train(const pack3d_desc *desc, const int32_t *coords, const void *q,
                         const void *k, const void *v, const void *gate, void *o, void *saved,
                         size_t saved_bytes, void *ws, size_t ws_bytes, void *stream,
                         void *const *stage_events);
#define PACK3D_NUM_BWD_STAGES 3
int pack3d_backward_workspace_bytes(const pack3d_desc *desc, size_t *bytes);
int pack3d_backward(const pack3d_desc *desc, const int32_t *coords, const void *q, const void *k,
                    const void *v, const void *gate, const void *saved, size_t saved_bytes,
                    const void *dout, void *dq, void *dk, void *dv, void *dgate, void *ws,
                    size_t ws_bytes, void *stream, void *const *stage_events);

#ifdef __cplusplus
}
#endif

#endif /* PACK3D_H */
