/*
 * tern.h -- C ABI of libtern, packed ternary (W1.58A16) linear layers on AMD
 * MI355X (gfx950).
 *
 * The operation.  A quantized linear weight W (N output rows x K inputs) is a
 * stack of trit planes T_p in {-1,0,+1}^{N x K} with one FP16 scale per
 * (row, group of G inputs), an optional FP16 offset, and residual planes that
 * exist only on salience-selected groups:
 *     W[n,k] = off(n,g) + sum_p m_p[n,g] * s_p[n,g] * T_p[n,k],  g = k / G,
 * and the library computes y[m,n] = sum_k W[n,k] * x[m,k] for FP16
 * activations x.  Sources: "Post-Training Ternarization of Qwen3-4B"
 * (arXiv 2609.01962v1 summary) §4.3 (offset plus ternary planes with
 * scales), §4.4 (salience masks select which weights get a second plane),
 * §4.5 (group size 128), §9.1 and §15 (persist the discrete planes and run a
 * lossless native kernel); arXiv 2609.09240 (Qwen3-8B scale-up),
 * representation, packing and direct-execution paragraphs.  The pages drop
 * the displayed reconstruction equation; the additive reading above is the
 * one this library implements.
 *
 * Packed layout (this library's definition; the pages print none):
 *   plane 0, TERN_FMT_2BIT: code(t) = t mod 4 (00 = 0, 01 = +1, 11 = -1; 10
 *     invalid).  Each little-endian uint32 holds 16 consecutive trits of a
 *     row; the trit at offset o occupies bits 16*(o%2) + 2*(o/2) .. +1 (even
 *     offsets in the low half-word, odd offsets in the high half-word).  Row
 *     stride K/4 bytes.
 *   plane 0, TERN_FMT_B3: every group of G trits takes ceil(G/5) bytes; byte
 *     j of a group is sum_i (t[5j+i]+1)*3^i, i = 0..4 (positions past the end
 *     of the group are zero trits).  Groups are consecutive; each row is
 *     zero-padded to a multiple of 16 bytes (tern_row_stride).
 *   residual plane p (1 or 2): mask[p-1] is a uint32 bitmap [N][ceil((K/G)/32)]
 *     (bit g%32 of word g/32 set when group g of row n carries plane p);
 *     rowptr[p-1] is [N+1] uint32, the exclusive prefix sum of the per-row
 *     popcounts; blocks[p-1] is [nnz][G/4] bytes, the 2-bit encoding of the G
 *     trits of each masked group in (row, group) order; rscale[p-1] is FP16
 *     [nnz] in the same order.
 *   scale0: FP16 [N][K/G].  offset: FP16 [N] (TERN_OFF_ROW) or [N][K/G]
 *     (TERN_OFF_GROUP), NULL for TERN_OFF_NONE.
 *
 * Conventions.
 *   - Every array argument is caller-owned device memory (e.g. from torch);
 *     the library allocates no device memory and keeps none between calls.
 *     Host-side descriptors (tern_matrix, arrays of them) are read during the
 *     call only.
 *   - Alignment (TERN_E_ALIGN otherwise): plane0, blocks, trits, x and
 *     workspaces 16 bytes (they are read with 16-byte vector loads); every
 *     other array its element size.
 *   - Supported shapes: n >= 0, k >= 0, k % 64 == 0, group % 64 == 0,
 *     group <= 1024, k % group == 0, 1 <= planes <= 3 (TERN_E_UNSUPPORTED
 *     otherwise).  n == 0 or m == 0 is an empty product and returns TERN_OK
 *     without touching memory; k == 0 writes y = 0.
 *   - x is [m][k] FP16, row-major; y is [m][n], row-major, FP16 (rounded to
 *     nearest even from an FP32 accumulator) or FP32.  y is overwritten.
 *   - stream is a hipStream_t (NULL = the null stream).  Products run
 *     asynchronously on it; launch failures return TERN_E_HIP and device
 *     faults surface at the caller's next synchronisation.  tern_pack and
 *     tern_unpack synchronise the stream so they can return validation
 *     results.
 *   - Products trust their packed input (no validation of codes); use
 *     tern_unpack to validate an artifact.
 *   - Errors are status codes; nothing throws across the ABI.
 *     tern_last_error() returns a message for the calling thread's last
 *     failure.
 */
#ifndef TERN_H
#define TERN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tern_status {
  TERN_OK = 0,
  TERN_E_INVAL = -1,        /* bad argument value, bad trit, trit outside mask */
  TERN_E_ALIGN = -2,        /* a device pointer is not 16-byte aligned */
  TERN_E_UNSUPPORTED = -3,  /* shape or mode outside the supported set */
  TERN_E_CORRUPT = -4,      /* packed bytes are not a valid encoding */
  TERN_E_WORKSPACE = -5,    /* workspace missing or too small */
  TERN_E_HIP = -6           /* a HIP runtime call failed */
} tern_status;

typedef enum tern_format { TERN_FMT_2BIT = 0, TERN_FMT_B3 = 1 } tern_format;
typedef enum tern_offset_mode { TERN_OFF_NONE = 0, TERN_OFF_ROW = 1, TERN_OFF_GROUP = 2 } tern_offset_mode;
typedef enum tern_dtype { TERN_F16 = 0, TERN_F32 = 1 } tern_dtype;

/* Indices of tern_packed_sizes' output array. */
typedef enum tern_buffer {
  TERN_BUF_PLANE0 = 0, TERN_BUF_SCALE0 = 1, TERN_BUF_OFFSET = 2, TERN_BUF_MASK = 3,
  TERN_BUF_ROWPTR = 4, TERN_BUF_BLOCKS1 = 5, TERN_BUF_BLOCKS2 = 6, TERN_BUF_RSCALE1 = 7,
  TERN_BUF_RSCALE2 = 8, TERN_NBUF = 9
} tern_buffer;

/* Host struct of caller-owned device pointers describing one packed matrix.
 * Members for absent residual planes and offsets are ignored (may be NULL). */
typedef struct tern_matrix {
  int32_t n, k, group, planes;   /* planes = 1 + number of residual planes */
  int32_t format;                /* tern_format of plane 0 */
  int32_t offset_mode;           /* tern_offset_mode */
  uint8_t  *plane0;              /* [n][tern_row_stride(k, group, format)] */
  uint16_t *scale0;              /* fp16 [n][k/group] */
  uint32_t *mask[2];             /* residual plane p: bitmap [n][ceil(k/group/32)] */
  uint32_t *rowptr[2];           /* [n+1] */
  uint8_t  *blocks[2];           /* [nnz[p-1]][group/4] */
  uint16_t *rscale[2];           /* fp16 [nnz[p-1]] */
  uint16_t *offset;              /* fp16 [n] or [n][k/group]; NULL for TERN_OFF_NONE */
  uint32_t nnz[2];               /* masked groups of residual planes 1 and 2 */
} tern_matrix;

/* Bytes per packed plane-0 row; 0 if (k, group, format) is unsupported. */
size_t tern_row_stride(int32_t k, int32_t group, int32_t format);

/* Host-only check of a descriptor (shapes, modes, NULL and alignment of the
 * pointers the product reads).  Makes no HIP call. */
tern_status tern_check(const tern_matrix *w);

/* Byte sizes of every buffer of a packed matrix, indexed by tern_buffer.
 * nnz may be NULL when planes == 1. */
tern_status tern_packed_sizes(int32_t n, int32_t k, int32_t group, int32_t format,
                              int32_t planes, const uint32_t *nnz, int32_t offset_mode,
                              size_t out_bytes[TERN_NBUF]);

/* Device workspace needed by tern_pack / tern_unpack / tern_gemv / tern_gemm
 * on this matrix with m activation rows (the maximum over the four).  A
 * decode product that is split along K keeps FP32 partials there and sums
 * them in split order with a second kernel.  Calls that overlap in time must
 * not share a workspace. */
size_t tern_workspace_bytes(const tern_matrix *w, int32_t m);

/* Pack trit planes (lossless serialisation: 2609.01962 §9.1, §15).
 *   trits        device int8 [planes][n][k]
 *   rscale_dense device fp16 [planes-1][n][k/group]: residual scales per group;
 *                entries outside the mask are ignored.  NULL if planes == 1.
 *   dst          descriptor whose shape, format, mask[] and nnz[] are inputs
 *                and whose plane0, rowptr[], blocks[] and rscale[] buffers
 *                are written (scale0 and offset are not touched).
 *   ws           device workspace of tern_workspace_bytes(dst, 1) bytes.
 * Synchronises stream.  TERN_E_INVAL if a trit is outside {-1,0,1}, a
 * residual trit is non-zero outside its mask, or nnz disagrees with the mask. */
tern_status tern_pack(const int8_t *trits, const uint16_t *rscale_dense, const tern_matrix *dst,
                      void *ws, size_t ws_bytes, void *stream);

/* Unpack to device int8 [planes][n][k] (zeros outside the residual masks) and
 * validate the artifact (the pages check an artifact before trusting it:
 * "Post-Training Ternarization of Qwen3-4B" §11.3, a checkpoint that was not
 * ternary was rejected by verification, and §9.2, a lossy packing that had
 * dropped a plane).  ws: tern_workspace_bytes(src, 1).  Synchronises stream.  TERN_E_CORRUPT on a 2-bit
 * code 10, a base-3 byte above 242, a non-zero base-3 padding trit or a
 * rowptr that disagrees with the mask popcounts. */
tern_status tern_unpack(const tern_matrix *src, int8_t *trits, void *ws, size_t ws_bytes,
                        void *stream);

/* y = x W^T for 1 <= m <= 63 (the direct ternary product of
 * "Can ternary LLMs hit 1.58 bits per weight", How It Works, and 2609.09240's
 * direct packed execution).  m == 0 is a no-op; m >= 64 is
 * TERN_E_UNSUPPORTED (use tern_gemm).  ws: tern_workspace_bytes(w, m).
 * Up to m = 4 (base-3), 5 (2-bit, group 128) or 4 (2-bit, group 64) the
 * decode kernels run (base-3: the matrix-core stream kernel with a separate
 * residual pass when the product holds at least tern_b3_min_stages stages,
 * the lane-per-row decode below that; K parts, when the product is too
 * small to fill the GPU, are summed by a second kernel); from there to
 * m = 32 the 16-row matrix-core product, whose tile table and reduce table
 * a small kernel writes into ws from a description passed by value; from
 * m = 33 the tiles of tern_gemm.  No route takes a table from host memory
 * (the one exception: a base-3 product large enough for the stream kernel,
 * whose item lists are copied from host memory like tern_gemv_batched's),
 * so a call can be captured into a HIP graph and replayed while x changes,
 * as long as ws stays the call's own. */
tern_status tern_gemv(const tern_matrix *w, const uint16_t *x, int32_t m, void *y,
                      int32_t y_dtype, void *ws, size_t ws_bytes, void *stream);

/* tern_gemv for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same product, with the workspace in a fixed device array inside the
 * library of TERN_NOALLOC_WORKSPACE_BYTES (16 MiB) per GPU, held by each GPU
 * the library runs on until the process ends.  Calls no hipMalloc or hipFree.
 * A product whose tern_workspace_bytes(w, m) exceeds that size returns
 * TERN_E_WORKSPACE (use tern_gemv with a workspace); 16 MiB covers every
 * m <= 63 product of the Qwen3-4B and -8B shapes.  Every call on a GPU uses
 * that GPU's one array: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.  The
 * remaining rules are tern_gemv's, graph capture included. */
#define TERN_NOALLOC_WORKSPACE_BYTES ((size_t)16 << 20)
tern_status tern_gemv_noalloc(const tern_matrix *w, const uint16_t *x, int32_t m, void *y,
                              int32_t y_dtype, void *stream);

/* y = x W^T for any m >= 0 through FP16 MFMA on tiles decoded into LDS
 * (tuned for m >= 64): the same direct product from the packed planes as
 * tern_gemv ("Post-Training Ternarization of Qwen3-4B" §10.2, a packed
 * kernel reading the encoded planes; 2609.09240's direct packed execution),
 * for many activation rows at once (prefill, batched decode; the pages
 * measure one row).  Supports group in {64, 128}; other groups return
 * TERN_E_UNSUPPORTED.  ws: tern_workspace_bytes(w, m) (unused today). */
tern_status tern_gemm(const tern_matrix *w, const uint16_t *x, int32_t m, void *y,
                      int32_t y_dtype, void *ws, size_t ws_bytes, void *stream);

/* Grouped product: count independent products y[i] = x[i] W[i]^T with the
 * same m, format, group and output dtype, in one launch (the layer's
 * projections of one token batch, say; the direct packed runtime of
 * 2609.09240 runs every linear layer of the model from its packed planes,
 * and this call runs a layer's, or a whole stack's, in one go), products
 * with the longest K first:
 *   m <= 4 (base-3), 5 (2-bit, group 128) or 4 (2-bit, group 64): the
 *     decode kernels.  2-bit: one workgroup per block of output rows, work
 *     items packed onto the CUs by size, products longer than a workgroup's
 *     activation stage cut into K parts.  Base-3, launches of at least
 *     tern_b3_min_stages stages: the activation layout and the residual pass
 *     (residual planes and offsets, FP32 row sums), then the persistent
 *     matrix-core stream kernel over 64-row items taken from per-XCD queues;
 *     products that read the same x (pointer and k) share its staged layout.
 *     Smaller base-3 launches: the lane-per-row decode, products of at least
 *     twice the shortest K cut into K parts;
 *   up to m = 32: FP16 MFMA on 16-row tiles decoded into LDS, K split into
 *     ranges of 4-step multiples;
 *   m >= 33: the matrix-core path of tern_gemm over every product's tiles,
 *     long-K products cut into K parts when that shortens the launch.
 *   A batch too small to fill the GPU has its decode products cut into
 *   more K parts.  K parts write FP32 partials to ws; on the decode kernels
 *   the last workgroup of each row block (arrival counters in ws, cleared
 *   by this call on stream) adds them in part order, on the matrix-core
 *   paths a second launch does; results are bitwise reproducible.
 *   w  host array [count] of descriptors
 *   x  host array [count] of device pointers, y likewise
 *   ws device workspace of tern_batch_workspace_bytes(w, count, m) bytes:
 *      the work tables (descriptors, per-workgroup records) are copied into
 *      it (hipMemcpyAsync on stream) on every call, and it holds the
 *      partials.  For repeated launches use tern_plan_create / tern_plan_run.
 * Products need k > 0 and group 64 or 128 (TERN_E_UNSUPPORTED otherwise). */
size_t tern_batch_workspace_bytes(const tern_matrix *w, int32_t count, int32_t m);
tern_status tern_gemv_batched(const tern_matrix *w, const uint16_t *const *x, void *const *y,
                              int32_t count, int32_t m, int32_t y_dtype, void *ws,
                              size_t ws_bytes, void *stream);

/* A prepared grouped product.  tern_plan_create copies the work tables into
 * the caller's device buffer `ws` of tern_batch_workspace_bytes bytes (which
 * also holds the plan's partials, arrival and queue counters -- cleared
 * here, and left clear by every run -- and the tables it derives from the
 * matrices; synchronously) and returns a host handle (malloc'ed; free it
 * with tern_plan_destroy).  tern_plan_run launches the whole batch on
 * stream; it may be called any number of times and captured in a HIP graph.
 * The buffers named in the plan must stay valid while the plan is used, and
 * their contents must not change in ways the plan has read: the plan keeps
 * tables derived from the masks, row pointers and residual scales (the
 * residual index, the residual pass's entry ranges, tile entry bounds) and,
 * for 2-bit products cut into K parts or with two residual planes, a copy
 * of the residual blocks in K-part order, so after a matrix is packed again
 * (or those arrays change) the plan must be created again; plane-0 bytes,
 * plane-0 scales, offsets and x may change between runs.  Runs of one plan (or of plans, or batched calls, that share a
 * workspace) use the same partials and counters, so runs that overlap in
 * time race: order them on one stream. */
typedef struct tern_plan tern_plan;
tern_status tern_plan_create(const tern_matrix *w, const uint16_t *const *x, void *const *y,
                             int32_t count, int32_t m, int32_t y_dtype, void *ws,
                             size_t ws_bytes, tern_plan **out);
tern_status tern_plan_run(const tern_plan *plan, void *stream);
/* tern_plan_run that also records two caller-created HIP events (hipEvent_t;
 * either may be NULL) on stream.  Base-3 plans at m <= 4: `before` behind
 * the launches that prepare the main decode's inputs (the activation layout
 * and the residual pass), `after` behind the main decode; the time between
 * them is that kernel's duration.  Other plans: the two bracket the whole
 * run.  A measurement hook; a run with events must not be captured in a
 * graph. */
tern_status tern_plan_run_events(const tern_plan *plan, void *stream, void *before, void *after);
void tern_plan_destroy(tern_plan *plan);
/* Kernel launches one tern_plan_run of this plan makes (rotation launches
 * included), for sizing graphs and reading traces; -1 for NULL.  Host-only,
 * no GPU call. */
int32_t tern_plan_launches(const tern_plan *plan);

/* A plan whose products take rotated activations: y[i] = x[i]
 * blockdiag(R_i)^T W[i]^T, the rotation applied to the activations before
 * the packed product ("Post-Training Ternarization of Qwen3-4B", §4.2: the
 * weights are quantized in a rotated basis and inference rotates the
 * activations to match), with R_i = rot[i] (device fp16
 * [k/rot_block][rot_block][rot_block], 16-byte aligned; NULL: product i
 * takes x[i] as it is), rot_block 64 or 128, each rotated k a multiple of
 * it; the rotation is that of tern_rotate (FP32 sums, FP16 values).
 * Products that read the same x must share its rotation (TERN_E_INVAL).
 * ws: tern_rotated_workspace_bytes(w, count, m) bytes; it holds the
 * counters of a rotation inside the product's launch (below), one rotated
 * copy of each distinct rotated x, then the plan's own tables.  Where the
 * rotation runs:
 *  - base-3 plans at m <= 4 on the stream kernel: inside their activation
 *    preparation (no launch of its own; the preparation then runs before the
 *    residual pass instead of alongside it);
 *  - 2-bit plans on the decode route (m <= 5 at group 128, m <= 4 at group
 *    64) with at most 8 distinct rotated inputs: inside the product's own
 *    launch, whose first workgroups rotate while the others request their
 *    first weights and then wait for the rotated activations (the FP32 sum
 *    of a rotated value is taken in an order of its own, so a value may
 *    differ from tern_rotate's in the last FP16 place);
 *  - other plans: rotation launches (tern_rotate_batched's kernel, up to 8
 *    inputs per launch) before the product.
 * tern_plan_launches tells which.  The counters make overlapping runs of one
 * plan race (as do its partial sums).  rot == NULL is tern_plan_create.  The
 * rest is as for tern_plan_create (run with tern_plan_run, free with
 * tern_plan_destroy). */
size_t tern_rotated_workspace_bytes(const tern_matrix *w, int32_t count, int32_t m);
tern_status tern_plan_create_rotated(const tern_matrix *w, const uint16_t *const *x,
                                     const uint16_t *const *rot, int32_t rot_block, void *const *y,
                                     int32_t count, int32_t m, int32_t y_dtype, void *ws,
                                     size_t ws_bytes, tern_plan **out);

/* Routing of base-3 products at m <= 4 (tern_gemv, tern_gemv_batched,
 * tern_plan_create and their workspace sizes).  A launch whose products
 * hold at least this many 64-row stages of plane 0 (ceil(n / 64) *
 * ceil(k / (8 * 128)) per product at group 128, ceil(k / (16 * 64)) at group
 * 64) runs the persistent matrix-core stream kernel with a separate residual
 * pass; smaller launches run the lane-per-row decode, whose work items are
 * finer.  Default: four stages per wavefront of the stream kernel at m = 1
 * (7168 on 256 CUs), four stages per CU at m = 2..4 (1024).  stages >= 0
 * sets one threshold for every m (0: every such launch takes the stream
 * kernel), -1 restores the defaults, any other negative value only queries.
 * Returns the threshold in effect before the call (the m = 1 one while the
 * defaults are in effect).  Process-wide;
 * workspace sizes and plans follow the threshold in effect when they are
 * computed or created.  Host-only. */
int64_t tern_b3_min_stages(int64_t stages);

/* Bits per weight of a packed matrix (2609.01962 §3.2, §7.1: effective bits
 * count log2(3) per stored trit over the planes actually present):
 *   info    = log2(3) * (n*k + group * sum nnz) / (n*k)
 *   plane   = 8 * (plane-0 bytes + residual block bytes) / (n*k)
 *   storage = 8 * (every byte of the representation) / (n*k)
 * Any output pointer may be NULL.  Host-only. */
tern_status tern_bits(const tern_matrix *w, double *info, double *plane, double *storage);

/* Quantizer front-end (the step before tern_pack): FP16 weights w [n][k]
 * -> trits [2][n][k] (int8, plane 0 then plane 1), scales [2][n][k/group]
 * (FP16) and per-group offsets [n][k/group] (FP16), so that
 *   W ~ offset + scales[0] * trits[0] + m * scales[1] * trits[1]
 * group by group (m: the group's bit in `mask`), ready for tern_pack with
 * planes = 2 and TERN_OFF_GROUP.  E2M-ATQ, order-2 asymmetric residual
 * ternarization ("Post-Training Ternarization of Qwen3-4B", §4.3): an offset
 * and two ternary planes with scales per group, then `iters` refinement
 * iterations (the pages use 15) with the ternary supports fixed; the second
 * plane only on the groups set in `mask` (salience-selected, §4.4; u32
 * bitmap [n][ceil(k/group/32)], bit g % 32 of word g / 32; NULL: none, and
 * trits[1] and scales[1] are zero).  Initial supports: |w - mean| > 0.7
 * mean|w - mean| (the ternary-weight-network threshold; the pages give no
 * rule); an iteration is the least-squares fit of (offset, s0, s1) followed
 * by the error-minimizing sign of every non-zero trit; a last fit gives the
 * stored values.  All arithmetic is FP32 in one fixed order, so results are
 * reproducible bit for bit.  group 64 or 128 and k % group == 0
 * (TERN_E_UNSUPPORTED otherwise); 0 <= iters <= 1000.  All pointers are
 * device memory owned by the caller (w, scales, offset 2-byte aligned, mask
 * 4-byte).  Async on stream. */
tern_status tern_quantize(const uint16_t *w, int32_t n, int32_t k, int32_t group, const uint32_t *mask,
                          int32_t iters, int8_t *trits, uint16_t *scales, uint16_t *offset, void *stream);

/* Activation-side rotation before the packed product ("Post-Training
 * Ternarization of Qwen3-4B", §4.2: the weights are quantized in a rotated
 * basis and inference rotates the activations to match; the pages do not
 * give the rotation's structure): out = x blockdiag(R)^T, i.e.
 *   out[m][b*block + i] = sum_j R[b][i][j] * x[m][b*block + j],
 * R fp16 [k/block][block][block] (16-byte aligned), x and out fp16 [m][k]
 * (4-byte aligned; out may equal x).  FP32 accumulation, FP16 output
 * (round to nearest even).  block 64 or 128 and k % block == 0
 * (TERN_E_UNSUPPORTED otherwise).  Async on stream. */
tern_status tern_rotate(const uint16_t *R, int32_t block, const uint16_t *x, int32_t m, int32_t k, uint16_t *out,
                        void *stream);

/* Several rotations in one launch (a layer's inputs, say): for i < count
 * (0..8; TERN_E_UNSUPPORTED above), out[i] = x[i] rotated by R[i] as in
 * tern_rotate, all with the same block and m; R, x, out are host arrays
 * of device pointers and k a host array of sizes (each a multiple of
 * block).  Inputs with k[i] == 0 are skipped (their pointers are not
 * read) and m == 0 launches nothing.  out[i] may equal x[i], but the
 * buffers of different inputs must not overlap.  No workspace: the
 * pointers travel in the kernel's arguments, so the call may be captured
 * into a HIP graph.  Async on stream. */
tern_status tern_rotate_batched(int32_t count, const uint16_t *const *R, int32_t block, const uint16_t *const *x,
                                const int32_t *k, int32_t m, uint16_t *const *out, void *stream);

/* Measurement aid, not part of the product: a plain streaming read of
 * `bytes` bytes (a multiple of 16) of device memory at `buf` (16-byte
 * aligned), the attainable-bandwidth reference for the products above.
 * `sink` is a device u32 that is written only for one improbable input
 * (it keeps the loads from being dropped).  Async on stream. */
tern_status tern_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream);

const char *tern_status_str(tern_status s);
const char *tern_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TERN_H */
