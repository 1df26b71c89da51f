// Host half of the C ABI declared in include/tern.h: argument and alignment
// checks, buffer and workspace sizing, work decomposition and launches.
#include "tern.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <queue>
#include <map>
#include <vector>

#include "internal.h"

using tern::GemvDesc;

namespace {

thread_local char g_err[512] = "";

tern_status fail(tern_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

tern_status hip_fail(hipError_t e, const char* what) {
  return fail(TERN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

tern_status tern::record_failure(tern_status s, const char* msg) { return fail(s, "%s", msg); }

namespace {

#define TERN_HIP(call)                                  \
  do {                                                  \
    hipError_t e_ = (call);                             \
    if (e_ != hipSuccess) return hip_fail(e_, #call);   \
  } while (0)

#define TERN_TRY(expr)                   \
  do {                                   \
    tern_status s_ = (expr);             \
    if (s_ != TERN_OK) return s_;        \
  } while (0)

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr size_t kFlagBytes = 256;
constexpr int kTargetItems = 512;   // decode workgroups (4 wavefronts each) that keep 256 CUs busy

tern_status check_shape(int32_t n, int32_t k, int32_t group, int32_t planes, int32_t format,
                        int32_t offset_mode) {
  if (n < 0 || k < 0) return fail(TERN_E_INVAL, "negative shape n=%d k=%d", n, k);
  if (group <= 0 || group % 64 || group > 1024)
    return fail(TERN_E_UNSUPPORTED, "group %d must be a positive multiple of 64 up to 1024", group);
  if (k % 64 || k % group) return fail(TERN_E_UNSUPPORTED, "k=%d must be a multiple of 64 and of group %d", k, group);
  if (planes < 1 || planes > 3) return fail(TERN_E_UNSUPPORTED, "planes=%d outside 1..3", planes);
  if (format != TERN_FMT_2BIT && format != TERN_FMT_B3) return fail(TERN_E_UNSUPPORTED, "unknown format %d", format);
  if (offset_mode < TERN_OFF_NONE || offset_mode > TERN_OFF_GROUP)
    return fail(TERN_E_UNSUPPORTED, "unknown offset mode %d", offset_mode);
  return TERN_OK;
}

// Arrays read with 16-byte vector loads (plane0, blocks, trits, x, workspace)
// need 16-byte alignment; the others need their element size.
tern_status check_dev(const void* p, bool needed, const char* name, size_t align = 16) {
  if (!p) return needed ? fail(TERN_E_INVAL, "%s is NULL", name) : TERN_OK;
  if (!aligned_to(p, align)) return fail(TERN_E_ALIGN, "%s is not %zu-byte aligned", name, align);
  return TERN_OK;
}

int mask_words(int k, int group) { return (k / group + 31) / 32; }

// Descriptor pointers that a product reads.
tern_status check_matrix(const tern_matrix* w) {
  if (!w) return fail(TERN_E_INVAL, "matrix descriptor is NULL");
  TERN_TRY(check_shape(w->n, w->k, w->group, w->planes, w->format, w->offset_mode));
  const bool body = w->n > 0 && w->k > 0;
  TERN_TRY(check_dev(w->plane0, body, "plane0"));
  TERN_TRY(check_dev(w->scale0, body, "scale0", 2));
  for (int p = 0; p < w->planes - 1; ++p) {
    TERN_TRY(check_dev(w->mask[p], body, "mask", 4));
    TERN_TRY(check_dev(w->rowptr[p], w->n > 0, "rowptr", 4));
    TERN_TRY(check_dev(w->blocks[p], body && w->nnz[p] > 0, "blocks"));
    TERN_TRY(check_dev(w->rscale[p], body && w->nnz[p] > 0, "rscale", 2));
    if ((uint64_t)w->nnz[p] > (uint64_t)w->n * (uint64_t)(w->k / w->group))
      return fail(TERN_E_INVAL, "nnz[%d]=%u exceeds the number of groups", p, w->nnz[p]);
  }
  TERN_TRY(check_dev(w->offset, body && w->offset_mode != TERN_OFF_NONE, "offset", 2));
  return TERN_OK;
}

// 2-bit products run on the matrix-core kernel, base-3 on the lane-per-row one.
bool use_mfma(int format) { return format == TERN_FMT_2BIT; }

int pick_mt(int m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8; }

// Activation rows per decode pass: 2-bit 8 (group 128) or 4 (group 64);
// base-3 4 (its LDS stage would not fit four wavefronts at 8 rows).
int max_mt(int format, int group) {
  return use_mfma(format) ? tern::gemv_mfma_max_rows(group) : 4;
}

// Groups on which K splits may start.
int split_quantum(int format, int group) {
  return use_mfma(format) ? std::max(1, 256 / group) : tern::gemv_stage_groups(format, group);
}

// Split of K into about `want` parts whose boundaries fall on split quanta;
// on the matrix-core kernel no part is longer than its activation stage.
void split_k(const tern_matrix* w, int want, int mp, int* splits, int* gps) {
  const int ng = w->k / w->group;
  const int sg = split_quantum(w->format, w->group);
  const int max_splits = std::max(1, (ng + sg - 1) / sg);
  const int s = std::min(max_splits, std::max(1, want));
  int g = (ng + s - 1) / s;
  g = (g + sg - 1) / sg * sg;
  g = std::max(g, sg);
  if (use_mfma(w->format)) {
    const int cap = std::max(sg, tern::gemv_mfma_max_range(mp) / w->group / sg * sg);
    g = std::min(g, cap);
  }
  *gps = g;
  *splits = std::max(1, (ng + g - 1) / g);
}

// Wavefronts sharing one 16-row tile's K on the matrix-core kernel: the
// fewest (1, 2 or 4) that keep each one's 256-trit blocks within 12 (all in
// flight at once) and near `ref`, so that long-K matrices of a batch finish
// with the short ones.
int choose_kwaves(int format, int k, int ref) {
  if (!use_mfma(format)) return 1;
  const int nblk = (k + 255) / 256, cap = std::min(std::max(ref, 8), 12);
  int kw = 1;
  while (kw < 4 && (nblk + kw - 1) / kw > cap) kw *= 2;
  return kw;
}

int rows_per_item(int kwaves) { return tern::kGemvRows / kwaves; }

// Single decode product: enough work items (row blocks x splits) to fill the GPU.
void choose_splits(const tern_matrix* w, int mp, int* splits, int* gps) {
  const int rpi = rows_per_item(choose_kwaves(w->format, w->k, 12));
  const int rb = std::max(1, (w->n + rpi - 1) / rpi);
  split_k(w, (kTargetItems + rb - 1) / rb, mp, splits, gps);
}

// Workspace of one split product: FP32 partials [splits][m][n].
size_t split_ws_bytes(int splits, int m, int n) {
  if (splits <= 1) return 0;
  return round_up((size_t)splits * m * n * sizeof(float), 256);
}

bool product_group_ok(int group) { return group == 64 || group == 128; }

int round256(int v) { return (v + 255) / 256 * 256; }

// Decode launch over descriptors (device table) or the single descriptor `one`.
hipError_t launch_decode(int format, int group, int mt, const GemvDesc* descs, const tern::WgRec* recs, int ndesc,
                         const GemvDesc& one, int items, int max_krp, bool offsets, hipStream_t s) {
  if (use_mfma(format)) return tern::launch_gemv_mfma(group, mt, descs, recs, ndesc, one, items, max_krp, offsets, s);
  return tern::launch_gemv(format, group, mt, descs, ndesc, one, items, s);
}

void fill_desc(GemvDesc& d, const tern_matrix* w, const uint16_t* x, int m, void* y, int y_f32) {
  std::memset(&d, 0, sizeof(d));
  d.plane0 = w->plane0;
  d.scale0 = w->scale0;
  for (int p = 0; p < 2; ++p) {
    const bool on = p < w->planes - 1;
    d.mask[p] = on ? w->mask[p] : nullptr;
    d.rowptr[p] = on ? w->rowptr[p] : nullptr;
    d.blocks[p] = on ? w->blocks[p] : nullptr;
    d.rscale[p] = on ? w->rscale[p] : nullptr;
    d.nnz[p] = on ? w->nnz[p] : 0u;
  }
  d.offset = w->offset_mode != TERN_OFF_NONE ? w->offset : nullptr;
  d.x = x;
  d.y = y;
  d.n = w->n;
  d.k = w->k;
  d.group = w->group;
  d.planes = w->planes;
  d.offset_mode = w->offset_mode;
  d.m = m;
  d.stride = (int32_t)tern_row_stride(w->k, w->group, w->format);
  d.ng = w->group ? w->k / w->group : 0;
  d.mwords = mask_words(w->k, w->group);
  d.splits = 1;
  d.gps = d.ng;
  d.row_blocks = (w->n + tern::kGemvRows - 1) / tern::kGemvRows;
  d.y_f32 = y_f32;
  d.kwaves = 1;
  d.ks0 = 0;
  d.ks1 = w->k / 64;
  d.kpart = -1;
}

void set_kwaves(GemvDesc& d, int kw) {
  d.kwaves = kw;
  d.row_blocks = (d.n + rows_per_item(kw) - 1) / rows_per_item(kw);
}

size_t gemv_ws_bytes(const tern_matrix* w, int m) {
  if (m <= 0 || w->n <= 0 || w->k <= 0 || !product_group_ok(w->group)) return 0;
  const int mc = std::min(m, max_mt(w->format, w->group));
  int splits, gps;
  choose_splits(w, pick_mt(mc), &splits, &gps);
  return split_ws_bytes(splits, mc, w->n);
}

tern_status flag_status(uint32_t flag, bool unpacking) {
  if (!flag) return TERN_OK;
  if (unpacking) {
    if (flag & tern::kFlagBadCode) return fail(TERN_E_CORRUPT, "invalid packed code (2-bit 10, base-3 byte > 242 or non-zero pad trit)");
    if (flag & tern::kFlagRowptr) return fail(TERN_E_CORRUPT, "rowptr disagrees with the mask popcounts");
    if (flag & tern::kFlagMaskBits) return fail(TERN_E_CORRUPT, "mask has bits past the last group");
  }
  if (flag & tern::kFlagBadTrit) return fail(TERN_E_INVAL, "trit outside {-1, 0, 1}");
  if (flag & tern::kFlagOutsideMask) return fail(TERN_E_INVAL, "non-zero residual trit outside its mask");
  if (flag & tern::kFlagMaskBits) return fail(TERN_E_INVAL, "mask has bits past the last group");
  return fail(TERN_E_INVAL, "validation flag 0x%x", flag);
}

tern_status check_xy(const uint16_t* x, void* y, int y_dtype) {
  if (y_dtype != TERN_F16 && y_dtype != TERN_F32) return fail(TERN_E_UNSUPPORTED, "unknown y dtype %d", y_dtype);
  TERN_TRY(check_dev(x, true, "x"));
  TERN_TRY(check_dev(y, true, "y", y_dtype == TERN_F32 ? 4 : 2));
  return TERN_OK;
}

}  // namespace

struct tern_plan {
  const GemvDesc* dev;    // one descriptor per work item / output tile, or the row ranges
  const tern::WgRec* recs;  // matrix-core decode: one record per workgroup (else NULL)
  int ndesc;              // descriptors at dev
  int total_items;
  int format, group, mt;
  int max_krp;
  bool offsets;
  bool gemm;              // m >= 33: grouped matrix-core product
  bool small;             // small m on the 16-row matrix-core product
  int aw, np;             // its activation tile (aw * 64 rows) and residual planes
  bool offs;              // some product has an offset
  const tern::RedDesc* red;  // small: split sums to reduce (device), their count and blocks
  int nred, red_blocks;
  bool b3;                // base-3 matrix-core decode: preparations, item lists and workgroups
  const tern::B3Prep* preps;
  int nprep;
  const tern::B3Item* b3items;
  uint32_t* queue;
  int nwg, b3_maxk;
  const tern::B3ResItem* b3res;  // residual pass units and their count
  int nres;
  bool prep_first;        // base-3: the preparations rotate, so they run before the residual pass
  tern::RotBatch* rots;   // rotations launched before the product (malloc'ed; NULL: none)
  int nrots, rot_block;
  bool folded;            // matrix-core decode: the rotations run inside its launch (fold)
  tern::RotFold fold;
};

extern "C" {

// Routing of products by activation rows (crossovers measured on an
// 8B-class layer on the MI355X): the decode kernels up to m = 4 (base-3,
// whose matrix-core decode covers four rows in one pass) or one 2-bit
// decode pass (m = 5 at group 128, where a pass holds 8 rows but
// the 16-row product wins from 6; m = 4 at group 64), the 16-row
// matrix-core product up to m = 32 (its time grows per 16 rows), the
// 128/256-row matrix-core tiles from m = 33.
static bool gemm_route(int m) { return m >= 33; }
static bool small_route(int format, int group, int m) {
  const int decode_max = format == TERN_FMT_B3 ? 4 : (group == 128 ? 5 : 4);
  return !gemm_route(m) && m > decode_max;
}
// Base-3 products with up to 4 activation rows run on the base-3 matrix-core
// decode (one pass covers 4 rows at the cost of one).
static bool b3_route(int format, int group, int m) {
  return format == TERN_FMT_B3 && product_group_ok(group) && m >= 1 && m <= 4;
}
// The same for a launch of count products: only launches with enough
// 64-row stages for the persistent stream kernel take it (defined with the
// base-3 batch builder).
static bool b3_route_n(const tern_matrix* w, int count, int m);

// Workspace of a small-m product batch (defined with the batch builder).
static size_t small_batch_ws_bytes(const tern_matrix* w, int32_t count, int32_t m);
// One small-m product whose tile table is written on the device (defined
// with the batch builder).
static tern_status small_gemv(const tern_matrix* w, const uint16_t* x, int32_t m, void* y, int32_t y_dtype,
                              void* ws, size_t ws_bytes, hipStream_t s);
// Single base-3 product at m <= 4 (defined with the base-3 batch builder).
static void b3_single_layout(const tern_matrix* w, int m, int* parts, int* sps, int* rsplit, size_t* x5_off,
                             size_t* xs_off, size_t* rp_off, size_t* rc_off, size_t* total);
static tern_status b3_gemv(const tern_matrix* w, const uint16_t* x, int32_t m, void* y, int32_t y_dtype, void* ws,
                           size_t ws_bytes, hipStream_t s);

size_t tern_row_stride(int32_t k, int32_t group, int32_t format) {
  if (k < 0 || group <= 0 || k % 64 || group % 64 || group > 1024 || k % group) return 0;
  if (format == TERN_FMT_2BIT) return (size_t)k / 4;
  if (format == TERN_FMT_B3) return round_up((size_t)(k / group) * ((group + 4) / 5), 16);
  return 0;
}

tern_status tern_check(const tern_matrix* w) { return check_matrix(w); }

tern_status tern_packed_sizes(int32_t n, int32_t k, int32_t group, int32_t format, int32_t planes,
                              const uint32_t* nnz, int32_t offset_mode, size_t out[TERN_NBUF]) {
  if (!out) return fail(TERN_E_INVAL, "out_bytes is NULL");
  TERN_TRY(check_shape(n, k, group, planes, format, offset_mode));
  if (planes > 1 && !nnz) return fail(TERN_E_INVAL, "nnz is NULL with residual planes");
  const size_t ng = (size_t)(k / group);
  for (int i = 0; i < TERN_NBUF; ++i) out[i] = 0;
  out[TERN_BUF_PLANE0] = (size_t)n * tern_row_stride(k, group, format);
  out[TERN_BUF_SCALE0] = (size_t)n * ng * 2;
  out[TERN_BUF_OFFSET] = offset_mode == TERN_OFF_ROW ? (size_t)n * 2 : offset_mode == TERN_OFF_GROUP ? (size_t)n * ng * 2 : 0;
  if (planes > 1) {
    out[TERN_BUF_MASK] = (size_t)n * mask_words(k, group) * 4;
    out[TERN_BUF_ROWPTR] = ((size_t)n + 1) * 4;
    for (int p = 0; p < planes - 1; ++p) {
      out[TERN_BUF_BLOCKS1 + p] = (size_t)nnz[p] * (group / 4);
      out[TERN_BUF_RSCALE1 + p] = (size_t)nnz[p] * 2;
    }
  }
  return TERN_OK;
}

size_t tern_workspace_bytes(const tern_matrix* w, int32_t m) {
  if (!w || check_shape(w->n, w->k, w->group, w->planes, w->format, w->offset_mode) != TERN_OK) return 0;
  const size_t packing = kFlagBytes + round_up(((size_t)w->n + 1) * 4, 256);
  size_t product = m > 0 && small_route(w->format, w->group, m) ? small_batch_ws_bytes(w, 1, m) : gemv_ws_bytes(w, m);
  if (b3_route_n(w, 1, m) && w->n > 0 && w->k > 0) {
    int parts, sps, rsplit;
    size_t x5_off, xs_off, rp_off, rc_off;
    b3_single_layout(w, m, &parts, &sps, &rsplit, &x5_off, &xs_off, &rp_off, &rc_off, &product);
  }
  return std::max(packing, product);
}

tern_status tern_pack(const int8_t* trits, const uint16_t* rscale_dense, const tern_matrix* dst,
                      void* ws, size_t ws_bytes, void* stream) {
  if (!dst) return fail(TERN_E_INVAL, "dst is NULL");
  TERN_TRY(check_shape(dst->n, dst->k, dst->group, dst->planes, dst->format, dst->offset_mode));
  const int n = dst->n, k = dst->k, group = dst->group;
  if (n == 0 || k == 0) return TERN_OK;
  TERN_TRY(check_dev(trits, true, "trits"));
  TERN_TRY(check_dev(dst->plane0, true, "plane0"));
  if (dst->planes > 1) TERN_TRY(check_dev(rscale_dense, true, "rscale_dense", 2));
  for (int p = 0; p < dst->planes - 1; ++p) {
    TERN_TRY(check_dev(dst->mask[p], true, "mask", 4));
    TERN_TRY(check_dev(dst->rowptr[p], true, "rowptr", 4));
    TERN_TRY(check_dev(dst->blocks[p], dst->nnz[p] > 0, "blocks"));
    TERN_TRY(check_dev(dst->rscale[p], dst->nnz[p] > 0, "rscale", 2));
  }
  if (!ws || ws_bytes < kFlagBytes) return fail(TERN_E_WORKSPACE, "pack needs %zu workspace bytes", kFlagBytes);
  TERN_TRY(check_dev(ws, true, "ws"));
  hipStream_t s = (hipStream_t)stream;
  uint32_t* flag = static_cast<uint32_t*>(ws);
  const int stride = (int)tern_row_stride(k, group, dst->format);
  const int ng = k / group, mw = mask_words(k, group);
  TERN_HIP(hipMemsetAsync(flag, 0, sizeof(uint32_t), s));
  TERN_HIP(tern::launch_pack_plane0(dst->format, trits, n, k, group, stride, dst->plane0, flag, s));
  for (int p = 0; p < dst->planes - 1; ++p) {
    const int8_t* tp = trits + (size_t)(p + 1) * n * k;
    TERN_HIP(tern::launch_mask_counts(dst->mask[p], n, ng, mw, dst->rowptr[p], flag, s));
    TERN_HIP(tern::launch_rowptr_scan(dst->rowptr[p], n, s));
    uint32_t total = 0, fl = 0;
    TERN_HIP(hipMemcpyAsync(&total, dst->rowptr[p] + n, sizeof(total), hipMemcpyDeviceToHost, s));
    TERN_HIP(hipMemcpyAsync(&fl, flag, sizeof(fl), hipMemcpyDeviceToHost, s));
    TERN_HIP(hipStreamSynchronize(s));
    if (fl) return flag_status(fl, false);
    if (total != dst->nnz[p])
      return fail(TERN_E_INVAL, "residual plane %d: mask has %u groups but nnz is %u", p + 1, total, dst->nnz[p]);
    TERN_HIP(tern::launch_pack_residual(tp, rscale_dense + (size_t)p * n * ng, dst->mask[p], dst->rowptr[p],
                                        n, k, group, mw, dst->blocks[p], dst->rscale[p], flag, s));
  }
  uint32_t fl = 0;
  TERN_HIP(hipMemcpyAsync(&fl, flag, sizeof(fl), hipMemcpyDeviceToHost, s));
  TERN_HIP(hipStreamSynchronize(s));
  return flag_status(fl, false);
}

tern_status tern_unpack(const tern_matrix* src, int8_t* trits, void* ws, size_t ws_bytes, void* stream) {
  TERN_TRY(check_matrix(src));
  const int n = src->n, k = src->k, group = src->group;
  if (n == 0 || k == 0) return TERN_OK;
  TERN_TRY(check_dev(trits, true, "trits"));
  const size_t need = kFlagBytes + round_up(((size_t)n + 1) * 4, 256);
  if (!ws || ws_bytes < need) return fail(TERN_E_WORKSPACE, "unpack needs %zu workspace bytes", need);
  TERN_TRY(check_dev(ws, true, "ws"));
  hipStream_t s = (hipStream_t)stream;
  uint32_t* flag = static_cast<uint32_t*>(ws);
  uint32_t* expect = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kFlagBytes);
  const int stride = (int)tern_row_stride(k, group, src->format);
  const int ng = k / group, mw = mask_words(k, group);
  TERN_HIP(hipMemsetAsync(flag, 0, sizeof(uint32_t), s));
  TERN_HIP(tern::launch_unpack_plane0(src->format, src->plane0, n, k, group, stride, trits, flag, s));
  for (int p = 0; p < src->planes - 1; ++p) {
    TERN_HIP(tern::launch_mask_counts(src->mask[p], n, ng, mw, expect, flag, s));
    TERN_HIP(tern::launch_rowptr_scan(expect, n, s));
    TERN_HIP(tern::launch_compare_u32(expect, src->rowptr[p], n + 1, tern::kFlagRowptr, flag, s));
    uint32_t total = 0, fl = 0;
    TERN_HIP(hipMemcpyAsync(&total, expect + n, sizeof(total), hipMemcpyDeviceToHost, s));
    TERN_HIP(hipMemcpyAsync(&fl, flag, sizeof(fl), hipMemcpyDeviceToHost, s));
    TERN_HIP(hipStreamSynchronize(s));
    if (fl & (tern::kFlagRowptr | tern::kFlagMaskBits)) return flag_status(fl, true);
    if (total != src->nnz[p])
      return fail(TERN_E_CORRUPT, "residual plane %d: mask has %u groups but nnz is %u", p + 1, total, src->nnz[p]);
    TERN_HIP(tern::launch_unpack_residual(src->blocks[p], src->mask[p], src->rowptr[p], n, k, group, mw,
                                          trits + (size_t)(p + 1) * n * k, flag, s));
  }
  uint32_t fl = 0;
  TERN_HIP(hipMemcpyAsync(&fl, flag, sizeof(fl), hipMemcpyDeviceToHost, s));
  TERN_HIP(hipStreamSynchronize(s));
  return flag_status(fl, true);
}

tern_status tern_gemv(const tern_matrix* w, const uint16_t* x, int32_t m, void* y, int32_t y_dtype,
                      void* ws, size_t ws_bytes, void* stream) {
  TERN_TRY(check_matrix(w));
  if (m < 0) return fail(TERN_E_INVAL, "m=%d is negative", m);
  if (m >= 64) return fail(TERN_E_UNSUPPORTED, "tern_gemv takes m <= 63 (got %d); use tern_gemm", m);
  if (m == 0 || w->n == 0) return TERN_OK;
  TERN_TRY(check_xy(x, y, y_dtype));
  if (!product_group_ok(w->group)) return fail(TERN_E_UNSUPPORTED, "products support group 64 or 128 (got %d)", w->group);
  hipStream_t s = (hipStream_t)stream;
  const int y_f32 = y_dtype == TERN_F32;
  GemvDesc d;
  fill_desc(d, w, x, m, y, y_f32);
  if (w->k == 0 || gemm_route(m)) {
    TERN_HIP(tern::launch_gemm(d, w->format, s));  // k == 0: zero fill
    return TERN_OK;
  }
  if (small_route(w->format, w->group, m)) return small_gemv(w, x, m, y, y_dtype, ws, ws_bytes, s);
  if (b3_route_n(w, 1, m)) return b3_gemv(w, x, m, y, y_dtype, ws, ws_bytes, s);
  const int cmax = max_mt(w->format, w->group);
  int splits, gps;
  choose_splits(w, pick_mt(std::min(m, cmax)), &splits, &gps);
  const size_t need = gemv_ws_bytes(w, m);
  if (need && (!ws || ws_bytes < need)) return fail(TERN_E_WORKSPACE, "tern_gemv needs %zu workspace bytes", need);
  if (need) TERN_TRY(check_dev(ws, true, "ws"));
  const size_t esz = y_f32 ? 4 : 2;
  set_kwaves(d, choose_kwaves(w->format, w->k, 12));
  for (int c0 = 0; c0 < m; c0 += cmax) {
    const int mc = std::min(cmax, m - c0);
    GemvDesc dc = d;
    dc.x = x + (size_t)c0 * w->k;
    dc.y = static_cast<char*>(y) + (size_t)c0 * w->n * esz;
    dc.m = mc;
    dc.splits = splits;
    dc.gps = gps;
    if (splits > 1) dc.partial = static_cast<float*>(ws);
    dc.tile_begin = 0;
    const int items = splits * dc.row_blocks;
    TERN_HIP(launch_decode(w->format, w->group, pick_mt(std::min(m, cmax)), nullptr, nullptr, 0, dc, items,
                           round256(gps * w->group), w->offset_mode != TERN_OFF_NONE, s));
    if (splits > 1) TERN_HIP(tern::launch_splitk_reduce(dc.partial, splits, mc, w->n, dc.y, y_f32, s));
  }
  return TERN_OK;
}

tern_status tern_gemm(const tern_matrix* w, const uint16_t* x, int32_t m, void* y, int32_t y_dtype,
                      void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  TERN_TRY(check_matrix(w));
  if (m < 0) return fail(TERN_E_INVAL, "m=%d is negative", m);
  if (m == 0 || w->n == 0) return TERN_OK;
  TERN_TRY(check_xy(x, y, y_dtype));
  if (!product_group_ok(w->group)) return fail(TERN_E_UNSUPPORTED, "products support group 64 or 128 (got %d)", w->group);
  GemvDesc d;
  fill_desc(d, w, x, m, y, y_dtype == TERN_F32);
  TERN_HIP(tern::launch_gemm(d, w->format, (hipStream_t)stream));
  return TERN_OK;
}

// CUs of the current device (256 on the MI355X when the query fails).
static int tern_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// Placement of the matrix-core decode work items.  The hardware hands
// workgroup j of a launch whose workgroups are all resident at once to the
// CU of workgroup j mod C (C CUs), so the item table is laid out by CU: the
// items are packed onto C bins (largest first, each onto the least loaded
// bin) and bin b's items take positions b, b + C, b + 2C, ...  Before that,
// while the launch has free slots, 64-row items are split into two 32-row
// items (twice the wavefronts per 16-row tile) so the bins can be evened
// out; a matrix keeps its 64-row items first and its 32-row items after
// them, as two row ranges.  Cost of an item: its 16-row x 256-trit blocks
// plus a fixed share for its prologue.
struct PlaceItem {
  int part, rb;
  long cost;
};

static tern_status place_balanced(const std::vector<GemvDesc>& parts, const std::vector<int>& pmat, int slots,
                                  std::vector<GemvDesc>* items, std::vector<int>* mat, std::vector<tern::WgRec>* recs) {
  const int cus = tern_cu_count();
  // coarse (current kwaves) and fine (twice the kwaves) items per part
  std::vector<int> coarse(parts.size()), fine(parts.size(), 0);
  long total = 0;
  // (row blocks; a part with K splits has that many items per row block)
  auto ns_of = [&](size_t t) { return (long)parts[t].splits; };
  for (size_t t = 0; t < parts.size(); ++t) {
    coarse[t] = parts[t].row_blocks;
    total += coarse[t] * ns_of(t);
  }
  auto rows_of = [&](size_t t, bool f) { return rows_per_item(parts[t].kwaves * (f ? 2 : 1)); };
  auto nblk_of = [&](size_t t) { return (long)((std::min(parts[t].k, parts[t].gps * parts[t].group) + 255) / 256); };
  auto fine_count = [&](size_t t, int a) {
    const int left = std::max(0, parts[t].n - a * rows_of(t, false));
    return (left + rows_of(t, true) - 1) / rows_of(t, true);
  };
  while (total < slots) {
    // split one 64-row item of the part whose coarse items cost the most
    long best = -1;
    size_t bt = 0;
    for (size_t t = 0; t < parts.size(); ++t) {
      if (parts[t].kwaves >= 4 || coarse[t] == 0) continue;
      const long c = (long)(rows_of(t, false) / 16) * nblk_of(t);
      if (c > best) { best = c; bt = t; }
    }
    if (best < 0) break;
    const int a = coarse[bt] - 1, f = fine_count(bt, a);
    const long grow = (a + f - (coarse[bt] + fine[bt])) * ns_of(bt);
    if (total + grow > slots) break;
    total += grow;
    coarse[bt] = a;
    fine[bt] = f;
  }
  // descriptors of the row ranges, and the items
  std::vector<GemvDesc> ranges;
  std::vector<int> rmat;
  std::vector<PlaceItem> all;
  for (size_t t = 0; t < parts.size(); ++t) {
    for (int f = 0; f < 2; ++f) {
      const int cnt = f ? fine[t] : coarse[t];
      if (cnt == 0) continue;
      GemvDesc d = parts[t];
      if (f) {
        set_kwaves(d, d.kwaves * 2);
        d.row_base = coarse[t] * rows_of(t, false);
      }
      d.row_blocks = cnt;
      const long tiles = rows_of(t, f != 0) / 16;
      // item = split * row_blocks + row block (the kernel's decomposition)
      for (int it = 0; it < cnt * d.splits; ++it) all.push_back(PlaceItem{(int)ranges.size(), it, tiles * nblk_of(t) + 4});
      ranges.push_back(d);
      rmat.push_back(pmat[t]);
    }
  }
  if (all.size() > (size_t)INT32_MAX || ranges.size() >= (1u << 12)) return fail(TERN_E_UNSUPPORTED, "batch too large");
  for (const PlaceItem& it : all)
    if (it.rb >= (1 << 20)) return fail(TERN_E_UNSUPPORTED, "batch too large");
  // largest first onto the least loaded bin
  std::stable_sort(all.begin(), all.end(), [](const PlaceItem& a, const PlaceItem& b) { return a.cost > b.cost; });
  std::vector<std::vector<int>> bins(cus);
  std::vector<long> load(cus, 0);
  typedef std::pair<long, int> LB;
  std::priority_queue<LB, std::vector<LB>, std::greater<LB>> heap;
  for (int b = 0; b < cus; ++b) heap.push(LB(0, b));
  for (size_t i = 0; i < all.size(); ++i) {
    const LB top = heap.top();
    heap.pop();
    bins[top.second].push_back((int)i);
    load[top.second] = top.first + all[i].cost;
    heap.push(LB(load[top.second], top.second));
  }
  // bins with more items take the lower CU numbers, so every round of C
  // positions is filled from its start
  std::vector<int> border(cus);
  for (int b = 0; b < cus; ++b) border[b] = b;
  std::stable_sort(border.begin(), border.end(), [&](int a, int b) { return bins[a].size() > bins[b].size(); });
  *items = ranges;
  if (mat) *mat = rmat;
  recs->clear();
  for (size_t round = 0;; ++round) {
    bool any = false;
    for (int r = 0; r < cus; ++r) {
      const std::vector<int>& bin = bins[border[r]];
      if (round >= bin.size()) break;
      const PlaceItem& it = all[bin[round]];
      tern::WgRec rec;
      std::memset(&rec, 0, sizeof(rec));
      rec.ri = (uint32_t)it.part << 20 | (uint32_t)it.rb;
      recs->push_back(rec);
      any = true;
    }
    if (!any) break;
  }
  return TERN_OK;
}

// ---- grouped decode
// The lane-per-row kernel reads one descriptor per work item (the
// descriptor of the (matrix, block of activation rows) the item belongs to,
// longest K first); the matrix-core kernel reads row-range descriptors and
// one record per workgroup.  Products cut into K parts (batch_splits) write
// FP32 partials [splits][m][n]; the last workgroup of each row block to
// finish (arrival counters in the workspace) sums them in part order and
// writes y, inside the same launch.
struct DecodeSplits {
  size_t partial_bytes = 0;
  size_t recs_off = 0;  // matrix-core decode: where the workgroup records start
  size_t part_off = 0;  // where the partials start
  size_t ctr_off = 0;   // where the arrival counters start (after the partials)
  size_t nctr = 0;      // counters: one per row block of each descriptor with K parts
};

// K parts of a 2-bit product on the matrix-core decode kernel at mp
// activation rows: a workgroup stages the activations of its K range, so a
// product longer than the stage holds is cut into parts (split_k), each with
// kwaves chosen for its own length.
static void mfma_split(const tern_matrix* w, int mp, int nblk_min, int* ns, int* gps, int* kw) {
  const int cap = tern::gemv_mfma_max_range(mp);
  *ns = 1;
  *gps = w->k / w->group;
  if (round256(w->k) > cap) split_k(w, (w->k + cap - 1) / cap, mp, ns, gps);
  *kw = choose_kwaves(w->format, std::min(w->k, *gps * w->group), nblk_min);
}

// Workspace offsets of a matrix-core decode batch with nparts (matrix, row
// chunk) parts and at most items_max workgroups: [row ranges (two per part)]
// [workgroup records][partials][reduce table].
static void mfma_offsets(size_t nparts, size_t items_max, size_t* recs_off, size_t* part_off) {
  *recs_off = round_up(2 * nparts * sizeof(GemvDesc), 256);
  *part_off = *recs_off + round_up(items_max * sizeof(tern::WgRec), 256);
}

// K parts of every product of a decode batch at mp padded activation rows
// (vectors indexed like w; products with n == 0 or k == 0 keep one part).
// Matrix-core kernel: parts no longer than the activation stage holds (with
// kwaves chosen per part); lane-per-row kernel: products of at least twice
// the shortest K are cut so that their items end with the others.  A batch
// whose work items cannot fill the GPU even at their finest (16-row items
// on the matrix-core kernel, where the placement may go that far; 64-row
// items otherwise) -- one or two products with few rows -- has every product
// cut further by the factor that brings it to the target: three workgroups
// per CU on the matrix-core kernel, kTargetItems / 2 on the lane-per-row one.
static void batch_splits(const tern_matrix* w, int count, int m, int mp, std::vector<int>* ns,
                         std::vector<int>* gps, std::vector<int>* kw) {
  ns->assign(count, 1);
  gps->assign(count, 0);
  kw->assign(count, 1);
  if (count <= 0) return;
  const bool mf = use_mfma(w[0].format);
  const long chunks = (m + max_mt(w[0].format, w[0].group) - 1) / max_mt(w[0].format, w[0].group);
  auto live = [&](int i) { return w[i].n > 0 && w[i].k > 0; };
  int kmin = 1 << 30, nblk_min = 1 << 30;
  for (int i = 0; i < count; ++i)
    if (live(i)) {
      kmin = std::min(kmin, w[i].k);
      nblk_min = std::min(nblk_min, (w[i].k + 255) / 256);
    }
  const int rows = mf ? tern::kGemvRows / 4 : tern::kGemvRows;
  long items = 0;
  for (int i = 0; i < count; ++i) {
    if (!live(i)) continue;
    (*gps)[i] = w[i].k / w[i].group;
    if (mf) mfma_split(&w[i], mp, nblk_min, &(*ns)[i], &(*gps)[i], &(*kw)[i]);
    else if (w[i].k >= 2 * kmin) split_k(&w[i], w[i].k / kmin, mp, &(*ns)[i], &(*gps)[i]);
    items += (long)((w[i].n + rows - 1) / rows) * (*ns)[i] * chunks;
  }
  // (measured: half as many lane-per-row items as a lone product's split
  // rule aims for finishes the small base-3 batches 2-3 % sooner)
#ifndef TERN_MFMA_TARGET  // workgroups per CU that a small matrix-core decode batch is cut to fill
#define TERN_MFMA_TARGET 3
#endif
  const long target = mf ? (long)TERN_MFMA_TARGET * tern_cu_count() : kTargetItems / 2;
  if (items == 0 || items >= target) return;
  const int f = (int)((target + items - 1) / items);
  for (int i = 0; i < count; ++i) {
    if (!live(i)) continue;
    split_k(&w[i], (*ns)[i] * f, mp, &(*ns)[i], &(*gps)[i]);
    if (mf) (*kw)[i] = choose_kwaves(w[i].format, std::min(w[i].k, (*gps)[i] * w[i].group), nblk_min);
  }
}

static tern_status build_batch(const tern_matrix* w, const uint16_t* const* x, void* const* y,
                               int32_t count, int32_t m, int32_t y_dtype, std::vector<GemvDesc>* items,
                               int* mt, int* max_krp, bool* offsets, std::vector<int>* mat,
                               std::vector<tern::WgRec>* recs, DecodeSplits* sp = nullptr, char* ws = nullptr) {
  if (count < 0) return fail(TERN_E_INVAL, "count=%d is negative", count);
  if (count > 0 && (!w || !x || !y)) return fail(TERN_E_INVAL, "NULL descriptor arrays");
  if (m < 0) return fail(TERN_E_INVAL, "m=%d is negative", m);
  if (y_dtype != TERN_F16 && y_dtype != TERN_F32) return fail(TERN_E_UNSUPPORTED, "unknown y dtype %d", y_dtype);
  items->clear();
  if (mat) mat->clear();
  recs->clear();
  *max_krp = 0;
  *offsets = false;
  std::vector<int> order;
  int nblk_min = 1 << 30;
  for (int i = 0; i < count; ++i) {
    TERN_TRY(check_matrix(&w[i]));
    if (w[i].format != w[0].format || w[i].group != w[0].group)
      return fail(TERN_E_UNSUPPORTED, "batched products must share format and group");
    if (!product_group_ok(w[i].group)) return fail(TERN_E_UNSUPPORTED, "products support group 64 or 128");
    if (w[i].n == 0 || m == 0) continue;
    if (w[i].k == 0) return fail(TERN_E_UNSUPPORTED, "batched decode needs k > 0");
    TERN_TRY(check_xy(x[i], y[i], y_dtype));
    order.push_back(i);
    nblk_min = std::min(nblk_min, (w[i].k + 255) / 256);
  }
  const int cmax = count > 0 ? max_mt(w[0].format, w[0].group) : 1;
  *mt = pick_mt(std::min(std::max(m, 1), cmax));
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a].k > w[b].k; });
  const size_t esz = y_dtype == TERN_F32 ? 4 : 2;
  std::vector<GemvDesc> parts;
  std::vector<int> pmat;
  for (int i : order) {
    for (int c0 = 0; c0 < m; c0 += cmax) {
      GemvDesc d;
      fill_desc(d, &w[i], x[i] + (size_t)c0 * w[i].k, std::min(cmax, m - c0),
                static_cast<char*>(y[i]) + (size_t)c0 * w[i].n * esz, y_dtype == TERN_F32);
      set_kwaves(d, choose_kwaves(w[i].format, w[i].k, nblk_min));
      parts.push_back(d);
      pmat.push_back(i);
      *max_krp = std::max(*max_krp, round256(w[i].k));
      *offsets = *offsets || w[i].offset_mode != TERN_OFF_NONE;
    }
  }
  std::vector<int> bns, bgps, bkw;
  batch_splits(w, count, m, *mt, &bns, &bgps, &bkw);
  if (count > 0 && use_mfma(w[0].format)) {
    // products cut into K parts write FP32 partials that the row blocks'
    // last workgroups sum in part order
    *max_krp = 0;
    size_t coarse_items = 0;
    for (size_t t = 0; t < parts.size(); ++t) {
      GemvDesc& d = parts[t];
      const int ns = bns[pmat[t]], g = bgps[pmat[t]];
      set_kwaves(d, bkw[pmat[t]]);
      d.splits = ns;
      d.gps = g;
      *max_krp = std::max(*max_krp, round256(std::min(d.k, g * d.group)));
      coarse_items += (size_t)d.row_blocks * ns;
    }
    const int slots = tern_cu_count() * std::min(tern::gemv_mfma_wgs_per_cu(w[0].group, *mt, *max_krp, *offsets),
                                                 tern::kMfmaMaxWgsPerCu);
    size_t recs_off, part_off;
    mfma_offsets(parts.size(), std::max(coarse_items, (size_t)slots), &recs_off, &part_off);
    size_t poff = 0;
    for (GemvDesc& d : parts) {
      if (d.splits <= 1) continue;
      if (!sp) return fail(TERN_E_UNSUPPORTED, "K parts need the workspace layout");
      d.partial = ws ? reinterpret_cast<float*>(ws + part_off + poff) : nullptr;
      poff += round_up((size_t)d.splits * d.m * d.n * 4, 256);
    }
    TERN_TRY(place_balanced(parts, pmat, slots, items, mat, recs));
    // one arrival counter per row block of every row range with K parts
    const size_t ctr_off = part_off + poff;
    size_t nctr = 0;
    for (GemvDesc& d : *items) {
      if (d.splits <= 1) continue;
      d.ctr = ws ? reinterpret_cast<uint32_t*>(ws + ctr_off) + nctr : nullptr;
      nctr += (size_t)d.row_blocks;
    }
    if (sp) {
      sp->partial_bytes = poff;
      sp->recs_off = recs_off;
      sp->part_off = part_off;
      sp->ctr_off = ctr_off;
      sp->nctr = nctr;
    }
    return TERN_OK;
  }
  // K parts of the products
  std::vector<int> nsp(parts.size(), 1), gps(parts.size(), 0);
  size_t nitems = 0;
  for (size_t t = 0; t < parts.size(); ++t) {
    nsp[t] = bns[pmat[t]];
    gps[t] = bgps[pmat[t]];
    if (nsp[t] > 1 && !sp) return fail(TERN_E_UNSUPPORTED, "K parts need the workspace layout");
    nitems += (size_t)parts[t].row_blocks * nsp[t];
  }
  if (nitems > (size_t)INT32_MAX) return fail(TERN_E_UNSUPPORTED, "batch too large");
  const size_t dbytes = round_up(nitems * sizeof(GemvDesc), 256);
  size_t ptotal = 0;
  for (size_t t = 0; t < parts.size(); ++t)
    if (nsp[t] > 1) ptotal += round_up((size_t)nsp[t] * parts[t].m * parts[t].n * 4, 256);
  const size_t ctr_off = dbytes + ptotal;
  size_t poff = 0, nctr = 0;
  for (size_t t = 0; t < parts.size(); ++t) {
    GemvDesc d = parts[t];
    d.tile_begin = (int)items->size();
    if (nsp[t] > 1) {
      // the row blocks' last K parts sum the partials (arrival counters)
      d.splits = nsp[t];
      d.gps = gps[t];
      d.partial = ws ? reinterpret_cast<float*>(ws + dbytes + poff) : nullptr;
      d.ctr = ws ? reinterpret_cast<uint32_t*>(ws + ctr_off) + nctr : nullptr;
      poff += round_up((size_t)nsp[t] * d.m * d.n * 4, 256);
      nctr += (size_t)d.row_blocks;
    }
    const size_t cnt = (size_t)d.row_blocks * nsp[t];
    items->insert(items->end(), cnt, d);
    if (mat) mat->insert(mat->end(), cnt, pmat[t]);
  }
  if (sp) {
    sp->partial_bytes = poff;
    sp->part_off = dbytes;
    sp->ctr_off = ctr_off;
    sp->nctr = nctr;
  }
  return TERN_OK;
}

// A batch of matrix-core tiles and its workspace layout:
// [descriptor per tile][FP32 partials of split products][reduce table].
struct TileBatch {
  std::vector<GemvDesc> tiles;
  std::vector<tern::RedDesc> red;
  size_t partial_bytes = 0;
  int red_blocks = 0, np = 0;
  bool offs = false;  // some product has an offset (with np, picks the tile decode's precision)
};

// ---- grouped matrix-core products (m >= 33)
// One descriptor per output tile (tile_rows x 128), matrices with the longest
// K first so that their tiles start first, and within a matrix the weight
// tile fastest.  np receives the most residual planes of any matrix.
// Split of each product's K (64-trit steps) for a grouped launch.  Three
// candidates: products whose tiles are at least twice as long as the
// shortest ones cut into that many parts; every product cut into parts of
// about 32 steps; and parts of about 16 steps (parts are multiples of 4 steps
// and at least 8).  Each candidate is scored by its makespan (largest tiles
// first onto the least-loaded of the resident slots, in steps) plus the time
// of its FP32 partials (written by the tiles, read by the grouped reduce)
// expressed in steps.  The best one is taken when it scores 15 % or more
// below the uncut launch.  The parts write FP32 partials that one grouped
// reduce sums in part order.
static std::vector<int> split_ranges(int steps, int parts) {
  std::vector<int> b(parts + 1, 0);
  const int q4 = (steps + 3) / 4;
  for (int i = 0; i <= parts; ++i) b[i] = std::min(steps, (int)((long)q4 * i / parts) * 4);
  b[parts] = steps;
  return b;
}

static long lpt_makespan(std::vector<long> len, int slots) {
  std::sort(len.begin(), len.end(), std::greater<long>());
  std::priority_queue<long, std::vector<long>, std::greater<long>> heap;
  for (int i = 0; i < std::max(1, slots); ++i) heap.push(0);
  long span = 0;
  for (long l : len) {
    const long t = heap.top() + l;
    heap.pop();
    heap.push(t);
    span = std::max(span, t);
  }
  return span;
}

// Measured time of one 64-trit step of a tile with one workgroup per CU
// (8B-class layer: 128-row tiles ~1.0 us, 256-row tiles ~1.7 us), and the
// rate at which partial sums are written and read back (~4 TB/s): together
// they turn a candidate's partial traffic into steps of launch time.
static double gemm_step_us(int bm) { return bm >= 256 ? 1.7 : 1.0; }
constexpr double kPartialBytesPerUs = 4.0e6;

static std::vector<int> gemm_splits(const tern_matrix* w, int32_t count, int32_t m) {
  std::vector<int> parts(count, 1);
  const int bm = tern::gemm_tile_rows(m);
  int smin = 1 << 30;
  for (int i = 0; i < count; ++i)
    if (w[i].n > 0 && w[i].k > 0) smin = std::min(smin, w[i].k / 64);
  if (smin == 1 << 30 || count == 0) return parts;
  const int slots = tern_cu_count() * tern::gemm_wgs_per_cu(w[0].format, bm / 64);
  // score of a split: makespan in steps plus the partial traffic in steps
  auto score = [&](const std::vector<int>& cut) {
    std::vector<long> len;
    double bytes = 0;
    for (int i = 0; i < count; ++i) {
      if (w[i].n <= 0 || w[i].k <= 0) continue;
      const long tiles = (long)((m + bm - 1) / bm) * ((w[i].n + 127) / 128);
      const std::vector<int> r = split_ranges(w[i].k / 64, cut[i]);
      for (int p = 0; p < cut[i]; ++p) len.insert(len.end(), tiles, r[p + 1] - r[p]);
      if (cut[i] > 1) bytes += 2.0 * cut[i] * (double)m * w[i].n * 4;
    }
    return (double)lpt_makespan(len, slots) + bytes / kPartialBytesPerUs / gemm_step_us(bm);
  };
  // parts of about `len` steps each (at least 8 steps, at most 8 parts)
  auto cut_to = [&](int len) {
    std::vector<int> c(count, 1);
    for (int i = 0; i < count; ++i) {
      if (w[i].n <= 0 || w[i].k <= 0) continue;
      const int st = w[i].k / 64;
      c[i] = std::max(1, std::min({8, st / 8, (st + len - 1) / len}));
    }
    return c;
  };
  std::vector<int> longc(count, 1);
  for (int i = 0; i < count; ++i) {
    if (w[i].n <= 0 || w[i].k <= 0) continue;
    const int st = w[i].k / 64;
    longc[i] = st >= 2 * smin ? std::min(8, st / smin) : 1;
    if (longc[i] > 1 && st / longc[i] < 8) longc[i] = std::max(1, st / 8);
  }
  const double plain = score(parts);
  double best = plain * 0.85;
  for (const std::vector<int>& cand : {longc, cut_to(32), cut_to(16)}) {
    const double sc = score(cand);
    if (sc <= best) {
      best = sc;
      parts = cand;
    }
  }
  return parts;
}

// Workgroup j of a launch runs on XCD j mod 8, and each XCD has its own L2.
// Each product's tiles (K part, then activation tile, weight tile fastest)
// are cut into 8 runs, run x for XCD x, so the workgroups of one XCD share
// activation tiles in its L2; every XCD takes the products longest K part
// first.  Positions a short XCD list leaves open hold empty descriptors
// (n = 0) that exit at once.
constexpr int kXcds = 8;

static size_t xcd_slots(const std::vector<size_t>& counts) {
  size_t len[kXcds] = {0};
  for (size_t t : counts)
    for (int x = 0; x < kXcds; ++x) len[x] += (x + 1) * t / kXcds - x * t / kXcds;
  size_t mx = 0;
  for (int x = 0; x < kXcds; ++x) mx = std::max(mx, len[x]);
  return mx * kXcds;
}

// One descriptor per output tile (tile_rows x 128) and K part, laid out by
// XCD as above.  With ws == nullptr only the layout is computed.
static tern_status build_gemm_batch(const tern_matrix* w, const uint16_t* const* x, void* const* y,
                                    int32_t count, int32_t m, int32_t y_dtype, char* ws, TileBatch* out) {
  if (count < 0) return fail(TERN_E_INVAL, "count=%d is negative", count);
  if (count > 0 && (!w || !x || !y)) return fail(TERN_E_INVAL, "NULL descriptor arrays");
  if (y_dtype != TERN_F16 && y_dtype != TERN_F32) return fail(TERN_E_UNSUPPORTED, "unknown y dtype %d", y_dtype);
  out->tiles.clear();
  out->red.clear();
  out->partial_bytes = 0;
  out->red_blocks = 0;
  out->np = 0;
  out->offs = false;
  std::vector<int> order;
  for (int i = 0; i < count; ++i) {
    TERN_TRY(check_matrix(&w[i]));
    if (w[i].format != w[0].format || w[i].group != w[0].group)
      return fail(TERN_E_UNSUPPORTED, "batched products must share format and group");
    if (!product_group_ok(w[i].group)) return fail(TERN_E_UNSUPPORTED, "products support group 64 or 128");
    if (w[i].n == 0) continue;
    if (w[i].k == 0) return fail(TERN_E_UNSUPPORTED, "batched products need k > 0");
    TERN_TRY(check_xy(x[i], y[i], y_dtype));
    order.push_back(i);
    out->np = std::max(out->np, w[i].planes - 1);
    out->offs = out->offs || w[i].offset_mode != TERN_OFF_NONE;
  }
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a].k > w[b].k; });
  const std::vector<int> parts = gemm_splits(w, count, m);
  const int bm = tern::gemm_tile_rows(m);
  std::vector<size_t> counts;
  for (int i : order) counts.push_back((size_t)parts[i] * ((m + bm - 1) / bm) * ((w[i].n + 127) / 128));
  const size_t ntiles = xcd_slots(counts);
  if (ntiles >= (size_t)INT32_MAX) return fail(TERN_E_UNSUPPORTED, "batch too large");
  const size_t tiles_bytes = round_up(ntiles * sizeof(GemvDesc), 256);
  std::vector<std::vector<GemvDesc>> ptiles;
  std::vector<int> plen;
  size_t poff = 0;
  for (int i : order) {
    GemvDesc d;
    fill_desc(d, &w[i], x[i], m, y[i], y_dtype == TERN_F32);
    const std::vector<int> r = split_ranges(w[i].k / 64, parts[i]);
    if (parts[i] > 1) {
      d.partial = ws ? reinterpret_cast<float*>(ws + tiles_bytes + poff) : nullptr;
      tern::RedDesc rd;
      rd.partial = d.partial;
      rd.y = y[i];
      rd.splits = parts[i];
      rd.m = m;
      rd.n = w[i].n;
      rd.y_f32 = y_dtype == TERN_F32;
      rd.begin = out->red_blocks;
      out->red.push_back(rd);
      out->red_blocks += (int)(((size_t)m * w[i].n + 255) / 256);
      poff += round_up((size_t)parts[i] * m * w[i].n * 4, 256);
    }
    ptiles.emplace_back();
    plen.push_back(0);
    for (int p = 0; p < parts[i]; ++p) {
      d.ks0 = r[p];
      d.ks1 = r[p + 1];
      d.kpart = parts[i] > 1 ? p : -1;
      plen.back() = std::max(plen.back(), r[p + 1] - r[p]);
      for (int tm = 0; tm < m; tm += bm)
        for (int tn = 0; tn < w[i].n; tn += 128) {
          d.tm0 = tm;
          d.tn0 = tn;
          ptiles.back().push_back(d);
        }
    }
  }
  std::vector<int> pord(ptiles.size());
  for (size_t j = 0; j < pord.size(); ++j) pord[j] = (int)j;
  std::stable_sort(pord.begin(), pord.end(), [&](int a, int b) { return plen[a] > plen[b]; });
  std::vector<std::vector<GemvDesc>> lists(kXcds);
  for (int j : pord) {
    const size_t t = ptiles[j].size();
    for (int x = 0; x < kXcds; ++x)
      lists[x].insert(lists[x].end(), ptiles[j].begin() + x * t / kXcds, ptiles[j].begin() + (x + 1) * t / kXcds);
  }
  GemvDesc none;
  std::memset(&none, 0, sizeof(none));
  out->tiles.assign(ntiles, none);
  for (int x = 0; x < kXcds; ++x)
    for (size_t r2 = 0; r2 < lists[x].size(); ++r2) out->tiles[r2 * kXcds + x] = lists[x][r2];
  out->partial_bytes = poff;
  return TERN_OK;
}

// Workspace of a grouped matrix-core batch, from the shapes alone.
static size_t gemm_batch_ws_bytes(const tern_matrix* w, int32_t count, int32_t m) {
  const std::vector<int> parts = gemm_splits(w, count, m);
  const int bm = tern::gemm_tile_rows(m);
  size_t partial = 0, nred = 0;
  std::vector<size_t> counts;
  for (int i = 0; i < count; ++i) {
    if (w[i].n <= 0 || w[i].k <= 0) continue;
    counts.push_back((size_t)parts[i] * ((m + bm - 1) / bm) * ((w[i].n + 127) / 128));
    if (parts[i] > 1) {
      partial += round_up((size_t)parts[i] * m * w[i].n * 4, 256);
      ++nred;
    }
  }
  return round_up(xcd_slots(counts) * sizeof(GemvDesc), 256) + partial + nred * sizeof(tern::RedDesc);
}

// ---- small m on the 16-row matrix-core product
// Decoded once per 16 activation rows, so the decode-bound small-m products
// keep the HBM stream; K is split into step ranges (64 trits per step,
// ranges a multiple of 4 steps) so that the grid holds about three workgroups
// per CU
// and no product's K runs long in one workgroup.  Unsplit tiles write y;
// split ones write FP32 partials that one grouped reduce sums in split order.


// Step ranges of a product with `steps` steps when the batch holds `total`
// tile-steps: a multiple of 4 steps each, at least 8, about total / (3 x CUs).
static std::vector<int> small_ranges(int steps, long total) {
  const long target = 3L * tern_cu_count();  // measured best: three workgroups per CU
  int u = (int)std::max<long>(8, (total / target + 3) / 4 * 4);
  const int nr = std::max(1, (steps + u - 1) / u);
  std::vector<int> b(nr + 1, 0);
  const int q4 = (steps + 3) / 4;  // ranges in units of 4 steps
  for (int i = 0; i <= nr; ++i) b[i] = std::min(steps, (int)((long)q4 * i / nr) * 4);
  b[nr] = steps;
  std::vector<int> out;
  for (int i = 0; i <= nr; ++i)
    if (out.empty() || b[i] > out.back() || i == nr) out.push_back(b[i]);
  return out;
}

// Layout of the workspace: [descriptor per tile][partials][reduce table].
static tern_status build_small_batch(const tern_matrix* w, const uint16_t* const* x, void* const* y, int32_t count,
                                     int32_t m, int32_t y_dtype, char* ws, TileBatch* out) {
  out->tiles.clear();
  out->red.clear();
  out->partial_bytes = 0;
  out->red_blocks = 0;
  out->np = 0;
  out->offs = false;
  std::vector<int> order;
  long total = 0;
  for (int i = 0; i < count; ++i) {
    TERN_TRY(check_matrix(&w[i]));
    if (w[i].format != w[0].format || w[i].group != w[0].group)
      return fail(TERN_E_UNSUPPORTED, "batched products must share format and group");
    if (!product_group_ok(w[i].group)) return fail(TERN_E_UNSUPPORTED, "products support group 64 or 128");
    if (w[i].n == 0) continue;
    if (w[i].k == 0) return fail(TERN_E_UNSUPPORTED, "batched products need k > 0");
    TERN_TRY(check_xy(x[i], y[i], y_dtype));
    order.push_back(i);
    out->np = std::max(out->np, w[i].planes - 1);
    out->offs = out->offs || w[i].offset_mode != TERN_OFF_NONE;
    total += (long)((w[i].n + 127) / 128) * (w[i].k / 64) * ((m + 15) / 16);
  }
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a].k > w[b].k; });
  const size_t esz = y_dtype == TERN_F32 ? 4 : 2;
  // partials first need their offsets: count them in a first pass
  size_t poff = 0;
  std::vector<std::pair<int, std::vector<int>>> plan;  // (matrix, ranges)
  for (int i : order) plan.push_back({i, small_ranges(w[i].k / 64, total)});
  const size_t tiles_bytes = [&] {
    size_t t = 0;
    for (auto& pr : plan)
      t += (size_t)((w[pr.first].n + 127) / 128) * (pr.second.size() - 1) * ((m + 15) / 16);
    return round_up(t * sizeof(GemvDesc), 256);
  }();
  for (auto& pr : plan) {
    const int i = pr.first;
    const std::vector<int>& rg = pr.second;
    const int nsplit = (int)rg.size() - 1;
    for (int c0 = 0; c0 < m; c0 += 16) {
      const int mc = std::min(16, m - c0);
      GemvDesc d;
      fill_desc(d, &w[i], x[i] + (size_t)c0 * w[i].k, mc, static_cast<char*>(y[i]) + (size_t)c0 * w[i].n * esz,
                y_dtype == TERN_F32);
      float* part = nullptr;
      if (nsplit > 1) {
        part = reinterpret_cast<float*>(ws + tiles_bytes + poff);
        tern::RedDesc r;
        r.partial = part;
        r.y = d.y;
        r.splits = nsplit;
        r.m = mc;
        r.n = w[i].n;
        r.y_f32 = y_dtype == TERN_F32;
        r.begin = out->red_blocks;
        out->red.push_back(r);
        out->red_blocks += (int)(((size_t)mc * w[i].n + 255) / 256);
        poff += round_up((size_t)nsplit * mc * w[i].n * 4, 256);
      }
      d.partial = part;
      for (int sp = 0; sp < nsplit; ++sp)
        for (int tn = 0; tn < w[i].n; tn += 128) {
          d.tn0 = tn;
          d.tm0 = rg[sp];
          d.splits = rg[sp + 1];
          d.gps = nsplit > 1 ? sp : -1;
          out->tiles.push_back(d);
        }
    }
  }
  out->partial_bytes = poff;
  return TERN_OK;
}

static size_t tile_ws_bytes(const TileBatch& b) {
  return round_up(b.tiles.size() * sizeof(GemvDesc), 256) + b.partial_bytes + b.red.size() * sizeof(tern::RedDesc);
}

// The same batch for one product, with the tiles and the reduce table
// written by a kernel from a compact description (launch_small_tiles), so
// that no table comes from host memory; a product with more K ranges than
// the description holds goes through tern_gemv_batched.
static tern_status small_gemv(const tern_matrix* w, const uint16_t* x, int32_t m, void* y, int32_t y_dtype,
                              void* ws, size_t ws_bytes, hipStream_t s) {
  if (!ws) return fail(TERN_E_WORKSPACE, "tern_gemv needs a workspace at m=%d", m);
  TERN_TRY(check_dev(ws, true, "ws"));
  TileBatch b;
  TERN_TRY(build_small_batch(w, &x, &y, 1, m, y_dtype, static_cast<char*>(ws), &b));
  if (b.tiles.empty()) return TERN_OK;
  const size_t need = tile_ws_bytes(b);
  if (ws_bytes < need) return fail(TERN_E_WORKSPACE, "tern_gemv needs %zu workspace bytes", need);
  tern::SmallSpec sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.nchunk = (m + 15) / 16;
  sp.ntn = (w->n + 127) / 128;
  sp.nsplit = (int)(b.tiles.size() / ((size_t)sp.nchunk * sp.ntn));
  bool fits = sp.nchunk <= 2 && b.red.size() <= 2 && sp.nsplit >= 1 && sp.nsplit <= tern::kSmallMaxRanges &&
              b.tiles.size() == (size_t)sp.nchunk * sp.nsplit * sp.ntn;
  if (fits) {
    for (int c = 0; c < sp.nchunk; ++c) sp.base[c] = b.tiles[(size_t)c * sp.nsplit * sp.ntn];
    for (int k = 0; k < sp.nsplit; ++k) {
      sp.rg[k] = b.tiles[(size_t)k * sp.ntn].tm0;
      sp.rg[k + 1] = b.tiles[(size_t)k * sp.ntn].splits;
    }
    sp.nred = (int)b.red.size();
    for (int r = 0; r < sp.nred; ++r) sp.red[r] = b.red[r];
    // the description reproduces the builder's table exactly
    for (size_t t = 0; t < b.tiles.size() && fits; ++t) {
      const int per = sp.nsplit * sp.ntn, c = (int)t / per, r = (int)t % per, k = r / sp.ntn;
      const GemvDesc& d = b.tiles[t];
      fits = d.tn0 == (r % sp.ntn) * 128 && d.tm0 == sp.rg[k] && d.splits == sp.rg[k + 1] &&
             d.gps == (sp.nsplit > 1 ? k : -1) && d.x == sp.base[c].x && d.y == sp.base[c].y &&
             d.partial == sp.base[c].partial && d.m == sp.base[c].m;
    }
  }
  if (!fits) {
    void* yp = y;
    return tern_gemv_batched(w, &x, &yp, 1, m, y_dtype, ws, ws_bytes, s);
  }
  char* base = static_cast<char*>(ws);
  const size_t tb = round_up(b.tiles.size() * sizeof(GemvDesc), 256);
  tern::RedDesc* red = reinterpret_cast<tern::RedDesc*>(base + tb + b.partial_bytes);
  TERN_HIP(tern::launch_small_tiles(sp, reinterpret_cast<GemvDesc*>(base), red, s));
  TERN_HIP(tern::launch_gemm_small(reinterpret_cast<const GemvDesc*>(base), (int)b.tiles.size(), w->format, w->group,
                                   b.np, b.offs, s));
  if (!b.red.empty()) TERN_HIP(tern::launch_reduce_grouped(red, (int)b.red.size(), b.red_blocks, s));
  return TERN_OK;
}

// Workspace of a small-m batch: the layout build_small_batch makes, from the
// shapes alone.
static size_t small_batch_ws_bytes(const tern_matrix* w, int32_t count, int32_t m) {
  long total = 0;
  for (int i = 0; i < count; ++i)
    if (w[i].n > 0 && w[i].k > 0) total += (long)((w[i].n + 127) / 128) * (w[i].k / 64) * ((m + 15) / 16);
  size_t tiles = 0, partial = 0, nred = 0;
  for (int i = 0; i < count; ++i) {
    if (w[i].n <= 0 || w[i].k <= 0) continue;
    const int nsplit = (int)small_ranges(w[i].k / 64, total).size() - 1;
    for (int c0 = 0; c0 < m; c0 += 16) {
      const int mc = std::min(16, m - c0);
      tiles += (size_t)nsplit * ((w[i].n + 127) / 128);
      if (nsplit > 1) {
        partial += round_up((size_t)nsplit * mc * w[i].n * 4, 256);
        ++nred;
      }
    }
  }
  return round_up(tiles * sizeof(GemvDesc), 256) + partial + nred * sizeof(tern::RedDesc);
}


// Plans of 2-bit products also keep a residual index after the descriptor
// table: per entry of the first residual plane, its group and scale (u32).
static bool plan_indexes(const tern_matrix* w) {
  return use_mfma(w->format) && w->planes == 2 && w->nnz[0] > 0 && w->n > 0 && w->k > 0;
}
static size_t index_bytes(const tern_matrix* w) { return plan_indexes(w) ? round_up((size_t)w->nnz[0] * 4, 256) : 0; }
// A plan also indexes per K part the residual planes of a matrix-core decode
// product cut into K parts or with two residual planes (GemvDesc::pidx), so
// that its items stage their entries as whole-row items do: the part row
// pointers, then the entries' blocks and index words.
static bool plan_part_indexes(const tern_matrix* w, int parts) {
  return use_mfma(w->format) && w->n > 0 && w->k > 0 && w->planes >= 2 && (parts > 1 || w->planes == 3) &&
         w->nnz[0] + (w->planes == 3 ? w->nnz[1] : 0u) > 0;
}
static size_t part_entries(const tern_matrix* w) { return (size_t)w->nnz[0] + (w->planes == 3 ? w->nnz[1] : 0u); }
static size_t part_index_bytes(const tern_matrix* w, int parts) {
  if (!plan_part_indexes(w, parts)) return 0;
  const size_t e = part_entries(w);
  return round_up(((size_t)parts * w->n + 1) * 4, 256) + round_up(e * (w->group / 4), 256) + round_up(e * 4, 256);
}

// ---- base-3 matrix-core decode batches (m <= 4)
// Workspace layout: [descriptors][activation preparations][queue counters]
// [items][residual pass units][partials of K-split products][arrival
// counters][x5 of each distinct activation][residual sums][residual index].
// The persistent launch (kB3Waves per CU) takes (product, 64-row block, K
// part) items, largest first, from a queue; a product is cut into K parts of
// whole 208-byte stages only when the launch would otherwise hold under two
// stages per wavefront, and into parts of at least two stages when it holds
// more stages than wavefronts.  Products that read the same activations (the same
// x pointer and k, as q/k/v or gate/up of a layer) share one x5.
struct B3Index {  // residual index of one plane of one product (launch_res_index)
  const uint32_t* mask;
  const uint32_t* rowptr;
  const uint16_t* rscale;
  int n, mwords;
  uint32_t* gidx;
};
struct B3Batch {
  std::vector<GemvDesc> descs;
  std::vector<B3Index> index;
  std::vector<tern::B3Prep> preps;
  std::vector<tern::B3Item> items;
  std::vector<tern::B3ResItem> res;  // residual pass units
  std::vector<uint32_t> queues;      // kB3Queues * kB3QueueWords words
  std::vector<std::pair<size_t, size_t>> zero;  // (offset, bytes) cleared at upload: residual-pass counters
  size_t rctr_off = 0, rctr_bytes = 0;
  bool prep_first = false;  // the preparations rotate (launched before the residual pass)
  size_t descs_off = 0, preps_off = 0, queue_off = 0, items_off = 0, part_off = 0, ctr_off = 0, res_off = 0, total = 0;
  size_t nctr = 0;
  int mt = 1, nwg = 0, max_k = 0;
};

static size_t b3_x5_bytes(const tern_matrix* w, int m) {
  return round_up((size_t)m * (w->k / w->group) * tern::b3_chunks_per_group(w->group) * 8, 256);
}
// 208-byte stages of a row.
static int b3_stages(const tern_matrix* w) {
  const int sg = tern::b3_stage_groups(w->group);
  return (w->k / w->group + sg - 1) / sg;
}
// Launches of fewer 64-row stages than this use the lane-per-row decode,
// whose work items are finer; tern_b3_min_stages changes it.  Default
// (measured on the MI355X): four per wavefront of the persistent launch at
// m = 1; four per CU at m = 2..4, where the lane-per-row decode holds more
// activation rows per lane (fewer wavefronts per SIMD) while the stream
// kernel covers up to four rows in one pass (4B- and 8B-class layers at m =
// 2..4: 7-30 % less time; single products of 256-768 stages stay faster
// on the lane-per-row decode).
static int64_t g_b3_min_stages = -1;
static int64_t b3_min_stages(int m = 1) {
  if (g_b3_min_stages >= 0) return g_b3_min_stages;
  return m >= 2 ? 4L * tern_cu_count() : 4L * tern_cu_count() * tern::kB3Waves;
}
static bool b3_route_n(const tern_matrix* w, int count, int m) {
  if (count <= 0 || !w || !b3_route(w[0].format, w[0].group, m)) return false;
  int64_t stages = 0;
  for (int i = 0; i < count; ++i)
    if (w[i].group == w[0].group && w[i].n > 0 && w[i].k > 0)
      stages += (int64_t)((w[i].n + tern::kGemvRows - 1) / tern::kGemvRows) * b3_stages(&w[i]);
  return stages >= b3_min_stages(m);
}
// A product with residual planes or an offset goes through the residual pass.
static bool b3_has_res(const tern_matrix* w) { return w->planes > 1 || w->offset_mode != TERN_OFF_NONE; }
static size_t b3_rsum_bytes(const tern_matrix* w, int m) {
  return b3_has_res(w) ? round_up((size_t)m * w->n * 4, 256) : 0;
}
static int b3_res_units(const tern_matrix* w) { return (w->n + tern::kB3ResRows - 1) / tern::kB3ResRows; }
// Residual pass: entry ranges per plane and row block (GemvDesc::rsplit) for
// the products `order` of w: up to about 2048 entries per unit, then more
// ranges (down to about 256 entries, one per thread) while the launch would
// hold fewer than two units per CU.
static std::vector<int> b3_res_splits(const tern_matrix* w, const std::vector<int>& order, int count) {
  std::vector<int> sp(count, 1);
  std::vector<double> avg(count, 0.0);
  long units = 0;
  for (int i : order) {
    if (!b3_has_res(&w[i])) continue;
    const int nrb = b3_res_units(&w[i]);
    for (int p = 0; p + 1 < w[i].planes; ++p) avg[i] = std::max(avg[i], (double)w[i].nnz[p] / nrb);
    sp[i] = std::max(1, (int)std::ceil(avg[i] / 2048.0));
    units += (long)nrb * std::max(1, w[i].planes - 1) * sp[i];
  }
  const long want = 2L * tern_cu_count();
  if (units > 0 && units < want) {
    const long f = (want + units - 1) / units;
    for (int i : order)
      if (b3_has_res(&w[i]) && w[i].planes > 1)
        sp[i] = (int)std::max<long>(sp[i], std::min<long>({(long)sp[i] * f, (long)(avg[i] / 256.0), 64L}));
  }
  return sp;
}
static int b3_res_slots(const tern_matrix* w, int split) { return w->planes > 1 ? (w->planes - 1) * split : 1; }
// Partial sums and arrival counters of a product whose residual pass has
// several units per row block.
static size_t b3_rpart_bytes(const tern_matrix* w, int m, int split) {
  return b3_has_res(w) && b3_res_slots(w, split) > 1 ? round_up((size_t)b3_res_slots(w, split) * m * w->n * 4, 256) : 0;
}
static size_t b3_rctr_bytes(const tern_matrix* w, int split) {
  return b3_has_res(w) && b3_res_slots(w, split) > 1 ? round_up((size_t)b3_res_units(w) * 4, 256) : 0;
}
// LDS a residual-pass workgroup may take.  Many units: a smaller window
// (more workgroups per CU).  Few units: 64 KB when that holds every group of
// the longest product in one window; when it cannot (the long product takes
// several windows either way), 52 KB for a third workgroup per CU as long as
// that window still holds 8 groups (8B-class layer at m = 4: 60.4 against
// 61.7 us; at m = 2, where 64 KB holds the whole down projection, 52 KB took
// 42.2 against 38.3 us).
static int b3_res_lds_cap(long nunits, int group, int mt, int max_k) {
  if (nunits > 4L * tern_cu_count()) return 36864;
  const int ng = group > 0 ? max_k / group : 0;
  if (ng <= 0 || tern::b3_res_window_groups(group, mt, max_k, 65536) >= ng) return 65536;
  return tern::b3_res_window_groups(group, mt, max_k, 53248) >= 8 ? 53248 : 65536;
}

// Builds the batch (items only when `items` is true); ws may be NULL (sizes only).
static tern_status build_b3_batch(const tern_matrix* w, const uint16_t* const* x, void* const* y, int32_t count,
                                  int32_t m, int32_t y_dtype, char* ws, bool items, B3Batch* b,
                                  const uint16_t* const* rot = nullptr, uint16_t* const* xr = nullptr,
                                  int rot_block = 0) {
  if (count < 0) return fail(TERN_E_INVAL, "count=%d is negative", count);
  if (count > 0 && !w) return fail(TERN_E_INVAL, "NULL descriptor array");
  if (items && count > 0 && (!x || !y)) return fail(TERN_E_INVAL, "NULL activation or output arrays");
  if (m < 1 || m > 4) return fail(TERN_E_UNSUPPORTED, "the base-3 decode takes 1..4 activation rows (m=%d)", m);
  if (y_dtype != TERN_F16 && y_dtype != TERN_F32) return fail(TERN_E_UNSUPPORTED, "unknown y dtype %d", y_dtype);
  b->mt = pick_mt(m);
  std::vector<int> order;
  for (int i = 0; i < count; ++i) {
    TERN_TRY(check_matrix(&w[i]));
    if (w[i].format != TERN_FMT_B3 || w[i].group != w[0].group)
      return fail(TERN_E_UNSUPPORTED, "batched products must share format and group");
    if (!product_group_ok(w[i].group)) return fail(TERN_E_UNSUPPORTED, "products support group 64 or 128");
    if (w[i].n == 0) continue;
    if (w[i].k == 0) return fail(TERN_E_UNSUPPORTED, "batched products need k > 0");
    if (items) TERN_TRY(check_xy(x[i], y[i], y_dtype));
    order.push_back(i);
  }
  const int cus = tern_cu_count();
  const long waves = (long)cus * tern::kB3Waves;
  // stages per K part: at most half the average stages per wavefront, but
  // two once the launch has more stages than wavefronts, so that an item's
  // second stage loads while its first decodes (8B-class layer, 2944 stages,
  // 1792 wavefronts: 62.3 against 72.8 us at m = 4, 38.4 against 44.5 us at
  // m = 2; three or four per part are slower)
  long units = 0;
  for (int i : order) units += (long)((w[i].n + tern::kGemvRows - 1) / tern::kGemvRows) * b3_stages(&w[i]);
  const int target = (int)std::max(units > waves ? 2L : 1L, units / (2 * waves));
  std::vector<int> sps(count, 1), parts(count, 1);
  size_t nres = 0;
  const std::vector<int> rsp = b3_res_splits(w, order, count);
  for (int i : order) {
    const int nst = b3_stages(&w[i]);
    sps[i] = std::min(nst, target);
    parts[i] = (nst + sps[i] - 1) / sps[i];
    b->max_k = std::max(b->max_k, w[i].k);
    if (b3_has_res(&w[i])) nres += (size_t)b3_res_units(&w[i]) * b3_res_slots(&w[i], rsp[i]);
  }
  // layout
  const size_t nd = order.size();
  b->descs_off = 0;
  b->preps_off = round_up(nd * sizeof(GemvDesc), 256);
  b->queue_off = b->preps_off + round_up(nd * sizeof(tern::B3Prep), 256);
  b->nwg = nd ? std::max(cus, tern::kB3Queues) : 0;
  b->items_off = b->queue_off + (size_t)tern::kB3Queues * tern::kB3QueueWords * 4;
  size_t nitems = 0, partial = 0, nctr = 0;
  for (int i : order) {
    const size_t rb = (size_t)(w[i].n + tern::kGemvRows - 1) / tern::kGemvRows;
    nitems += rb * parts[i];
    if (parts[i] > 1) {
      partial += round_up((size_t)parts[i] * m * w[i].n * 4, 256);
      nctr += rb;
    }
  }
  b->res_off = b->items_off + round_up(nitems * sizeof(tern::B3Item), 256);
  b->part_off = b->res_off + round_up(nres * sizeof(tern::B3ResItem), 256);
  b->ctr_off = b->part_off + partial;
  b->nctr = nctr;
  size_t off = b->ctr_off + round_up(nctr * 4, 256);
  // x5 per distinct activation (without x, as for sizing, one per product)
  std::vector<size_t> x5_off(count, 0), xs_off(count, 0);
  std::vector<bool> x5_own(count, true);
  std::map<std::pair<const uint16_t*, int>, int> x5_first;
  for (int i : order) {
    if (x) {
      auto ins = x5_first.insert({{x[i], w[i].k}, i});
      if (!ins.second) {
        const int f = ins.first->second;
        if (rot && rot[f] != rot[i])
          return fail(TERN_E_INVAL, "products %d and %d read the same x with different rotations", f, i);
        x5_off[i] = x5_off[f];
        x5_own[i] = false;
        continue;
      }
    }
    x5_off[i] = off;
    off += b3_x5_bytes(&w[i], m);
  }
  std::vector<size_t> rp_off(count, 0), rc_off(count, 0);
  for (int i : order) {
    xs_off[i] = off;  // residual sums
    off += b3_rsum_bytes(&w[i], m);
    rp_off[i] = off;  // residual pass partials and arrival counters
    off += b3_rpart_bytes(&w[i], m, rsp[i]);
    rc_off[i] = off;
    off += b3_rctr_bytes(&w[i], rsp[i]);
  }

  // residual index per plane (entry -> group and scale)
  std::vector<size_t> gi_off(2 * (size_t)count, 0);
  for (int i : order)
    for (int p = 0; p + 1 < w[i].planes; ++p) {
      gi_off[2 * i + p] = off;
      off += round_up((size_t)w[i].nnz[p] * 4, 256);
    }
  b->total = off;
  b->descs.clear();
  b->res.clear();
  b->zero.clear();
  b->prep_first = false;
  b->index.clear();
  b->preps.clear();
  b->items.clear();
  if (!items) return TERN_OK;

  // descriptors and preparations
  const size_t esz = y_dtype == TERN_F32 ? 4 : 2;
  (void)esz;
  size_t poff = 0, coff = 0;
  for (int i : order) {
    GemvDesc d;
    fill_desc(d, &w[i], rot && rot[i] ? xr[i] : x[i], m, y[i], y_dtype == TERN_F32);
    d.splits = parts[i];
    d.p0 = parts[i];
    d.gps = sps[i];
    d.x5 = ws ? reinterpret_cast<const uint16_t*>(ws + x5_off[i]) : nullptr;
    d.rsum = ws && b3_has_res(&w[i]) ? reinterpret_cast<const float*>(ws + xs_off[i]) : nullptr;
    d.rsplit = rsp[i];
    d.rslots = b3_res_slots(&w[i], rsp[i]);
    if (b3_has_res(&w[i]) && d.rslots > 1) {
      d.rpart = ws ? reinterpret_cast<float*>(ws + rp_off[i]) : nullptr;
      d.rctr = ws ? reinterpret_cast<uint32_t*>(ws + rc_off[i]) : nullptr;
      b->zero.push_back({rc_off[i], b3_rctr_bytes(&w[i], rsp[i])});
    }
    if (b3_has_res(&w[i]))
      for (int u = 0; u < b3_res_units(&w[i]); ++u)
        for (int sl = 0; sl < d.rslots; ++sl)
          b->res.push_back({(uint32_t)b->descs.size(), (uint32_t)u, (uint32_t)sl, 0u, 0u});
    for (int p = 0; p + 1 < w[i].planes; ++p) {
      uint32_t* gidx = ws ? reinterpret_cast<uint32_t*>(ws + gi_off[2 * i + p]) : nullptr;
      d.gidx[p] = gidx;
      if (w[i].nnz[p] > 0)
        b->index.push_back({w[i].mask[p], w[i].rowptr[p], w[i].rscale[p], w[i].n, mask_words(w[i].k, w[i].group), gidx});
    }
    if (parts[i] > 1) {
      d.partial = ws ? reinterpret_cast<float*>(ws + b->part_off + poff) : nullptr;
      d.ctr = ws ? reinterpret_cast<uint32_t*>(ws + b->ctr_off) + coff : nullptr;
      poff += round_up((size_t)parts[i] * m * w[i].n * 4, 256);
      coff += (size_t)d.row_blocks;
    }
    b->descs.push_back(d);
    if (!x5_own[i]) continue;
    tern::B3Prep pr;
    std::memset(&pr, 0, sizeof(pr));
    pr.x = x[i];
    pr.x5 = const_cast<uint16_t*>(d.x5);
    pr.k = w[i].k;
    pr.m = m;
    if (rot && rot[i]) {  // rotated in the preparation; the residual pass reads the rotated copy
      pr.R = rot[i];
      pr.xr = xr[i];
      pr.rblock = rot_block;
      b->prep_first = true;
    }
    b->preps.push_back(pr);
  }
  // residual units of the longest products first (workgroups start in
  // index order, so the longest activation stagings do not form the tail;
  // 8B-class stack: 409 against 413 us per token)
  std::stable_sort(b->res.begin(), b->res.end(), [&](const tern::B3ResItem& u, const tern::B3ResItem& v) {
    return b->descs[u.desc].k > b->descs[v.desc].k;
  });
  // items, largest first onto the least loaded wavefront
  struct It {
    uint32_t dp, rb;
    int cost;
  };
  std::vector<It> all;
  all.reserve(nitems);
  for (size_t di = 0; di < nd; ++di) {
    const GemvDesc& d = b->descs[di];
    const int nst = (d.ng + tern::b3_stage_groups(d.group) - 1) / tern::b3_stage_groups(d.group);
    for (int pt = 0; pt < d.splits; ++pt) {
      const int st = std::min(nst, (pt + 1) * d.gps) - pt * d.gps;
      for (int rb = 0; rb < d.row_blocks; ++rb) {
        const int rows = std::min(tern::kGemvRows, d.n - rb * tern::kGemvRows);
        const int cost = st * 64 + rows;
        all.push_back({(uint32_t)(di << 16 | (uint32_t)pt), (uint32_t)rb, cost});
      }
    }
  }
  if (nd > 65535) return fail(TERN_E_UNSUPPORTED, "a batch takes at most 65535 products");
  // largest first onto the queue (XCD) of least cost; each list stays in
  // decreasing cost, the order its wavefronts take them in
  std::stable_sort(all.begin(), all.end(), [](const It& a, const It& c) { return a.cost > c.cost; });
  std::vector<std::vector<uint32_t>> lists(tern::kB3Queues);
  std::vector<long> load(tern::kB3Queues, 0L);
  for (size_t t = 0; t < all.size(); ++t) {
    const int q = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    lists[q].push_back((uint32_t)t);
    load[q] += all[t].cost;
  }
  b->items.reserve(all.size());
  b->queues.assign((size_t)tern::kB3Queues * tern::kB3QueueWords, 0u);
  for (int q = 0; q < tern::kB3Queues; ++q) {
    b->queues[(size_t)q * tern::kB3QueueWords + 2] = (uint32_t)b->items.size();
    for (uint32_t t : lists[q]) b->items.push_back({all[t].dp, all[t].rb});
    b->queues[(size_t)q * tern::kB3QueueWords + 3] = (uint32_t)b->items.size();
  }
  return TERN_OK;
}

// Copies a built batch's tables into ws (asynchronously on s, or synchronously
// when s is NULL and sync is true) and clears its counters.
static tern_status upload_b3_batch(const B3Batch& b, char* ws, hipStream_t s, bool sync) {
  auto cp = [&](size_t off, const void* src, size_t bytes) -> hipError_t {
    if (!bytes) return hipSuccess;
    return sync ? hipMemcpy(ws + off, src, bytes, hipMemcpyHostToDevice)
                : hipMemcpyAsync(ws + off, src, bytes, hipMemcpyHostToDevice, s);
  };
  TERN_HIP(cp(b.descs_off, b.descs.data(), b.descs.size() * sizeof(GemvDesc)));
  TERN_HIP(cp(b.preps_off, b.preps.data(), b.preps.size() * sizeof(tern::B3Prep)));
  TERN_HIP(cp(b.items_off, b.items.data(), b.items.size() * sizeof(tern::B3Item)));
  TERN_HIP(cp(b.res_off, b.res.data(), b.res.size() * sizeof(tern::B3ResItem)));
  TERN_HIP(cp(b.queue_off, b.queues.data(), b.queues.size() * 4));
  for (const auto& z : b.zero)
    TERN_HIP(sync ? hipMemset(ws + z.first, 0, z.second) : hipMemsetAsync(ws + z.first, 0, z.second, s));
  if (b.nctr) TERN_HIP(sync ? hipMemset(ws + b.ctr_off, 0, b.nctr * 4) : hipMemsetAsync(ws + b.ctr_off, 0, b.nctr * 4, s));
  for (const B3Index& ix : b.index)
    TERN_HIP(tern::launch_res_index(ix.mask, ix.rowptr, ix.rscale, ix.n, ix.mwords, ix.gidx, sync ? nullptr : s));
  TERN_HIP(tern::launch_b3_res_ranges(reinterpret_cast<const GemvDesc*>(ws + b.descs_off),
                                      reinterpret_cast<tern::B3ResItem*>(ws + b.res_off), (int)b.res.size(),
                                      sync ? nullptr : s));
  if (sync && (!b.index.empty() || !b.res.empty())) TERN_HIP(hipStreamSynchronize(nullptr));
  return TERN_OK;
}

static tern_status run_b3_batch(const B3Batch& b, int group, char* ws, hipStream_t s) {
  if (b.descs.empty()) return TERN_OK;
  tern::B3Prep none;
  std::memset(&none, 0, sizeof(none));
  GemvDesc dummy;
  std::memset(&dummy, 0, sizeof(dummy));
  const tern::B3Prep* preps = reinterpret_cast<const tern::B3Prep*>(ws + b.preps_off);
  if (b.res.empty())
    TERN_HIP(tern::launch_b3_prep(group, preps, (int)b.preps.size(), none, b.max_k, s));
  else  // the preparations ride along in the residual pass's launch
    TERN_HIP(tern::launch_b3_res(group, b.mt, reinterpret_cast<const GemvDesc*>(ws + b.descs_off),
                                 reinterpret_cast<const tern::B3ResItem*>(ws + b.res_off), (int)b.res.size(), dummy,
                                 b.max_k, b3_res_lds_cap((long)b.res.size(), group, b.mt, b.max_k), preps,
                                 (int)b.preps.size(), b.max_k, s));
  TERN_HIP(tern::launch_gemv_b3(group, b.mt, reinterpret_cast<const GemvDesc*>(ws + b.descs_off),
                                reinterpret_cast<const tern::B3Item*>(ws + b.items_off),
                                reinterpret_cast<uint32_t*>(ws + b.queue_off), b.nwg, dummy,
                                (int)b.items.size(), s));
  return TERN_OK;
}

// Single base-3 product at m <= 4 without host tables: every wavefront takes
// items w, w + W, ... of the one descriptor; K parts (when the product is too
// small to fill the GPU) write FP32 partials that a second kernel sums.
// Workspace: [partials][x5][group sums].
static void b3_single_layout(const tern_matrix* w, int m, int* parts, int* sps, int* rsplit, size_t* x5_off,
                             size_t* xs_off, size_t* rp_off, size_t* rc_off, size_t* total) {
  const long waves = (long)tern_cu_count() * tern::kB3Waves;
  const int rb = (w->n + tern::kGemvRows - 1) / tern::kGemvRows;
  const int nst = b3_stages(w);
  const int target = (int)std::max(1L, (long)rb * nst / (2 * waves));
  *sps = std::min(nst, target);
  *parts = (nst + *sps - 1) / *sps;
  *rsplit = b3_res_splits(w, std::vector<int>{0}, 1)[0];
  *x5_off = split_ws_bytes(*parts, m, w->n);
  *xs_off = *x5_off + b3_x5_bytes(w, m);  // residual sums
  *rp_off = *xs_off + b3_rsum_bytes(w, m);  // residual pass partials, arrival counters
  *rc_off = *rp_off + b3_rpart_bytes(w, m, *rsplit);
  *total = *rc_off + b3_rctr_bytes(w, *rsplit);
  for (int p = 0; p + 1 < w->planes; ++p) *total += round_up((size_t)w->nnz[p] * 4, 256);  // residual index
}

static tern_status b3_gemv(const tern_matrix* w, const uint16_t* x, int32_t m, void* y, int32_t y_dtype, void* ws,
                           size_t ws_bytes, hipStream_t s) {
  int parts, sps, rsplit;
  size_t x5_off, xs_off, rp_off, rc_off, total;
  b3_single_layout(w, m, &parts, &sps, &rsplit, &x5_off, &xs_off, &rp_off, &rc_off, &total);
  if (!ws || ws_bytes < total) return fail(TERN_E_WORKSPACE, "tern_gemv needs %zu workspace bytes", total);
  TERN_TRY(check_dev(ws, true, "ws"));
  char* base = static_cast<char*>(ws);
  GemvDesc d;
  fill_desc(d, w, x, m, y, y_dtype == TERN_F32);
  d.splits = parts;
  d.p0 = parts;
  d.gps = sps;
  d.x5 = reinterpret_cast<const uint16_t*>(base + x5_off);
  d.rsum = b3_has_res(w) ? reinterpret_cast<const float*>(base + xs_off) : nullptr;
  d.rsplit = rsplit;
  d.rslots = b3_res_slots(w, rsplit);
  if (d.rsum && d.rslots > 1) {
    d.rpart = reinterpret_cast<float*>(base + rp_off);
    d.rctr = reinterpret_cast<uint32_t*>(base + rc_off);
  }
  if (parts > 1) d.partial = reinterpret_cast<float*>(base);
  size_t gi = rc_off + b3_rctr_bytes(w, rsplit);
  for (int p = 0; p + 1 < w->planes; ++p) {
    d.gidx[p] = reinterpret_cast<const uint32_t*>(base + gi);
    if (w->nnz[p] > 0)
      TERN_HIP(tern::launch_res_index(w->mask[p], w->rowptr[p], w->rscale[p], w->n, mask_words(w->k, w->group),
                                      reinterpret_cast<uint32_t*>(base + gi), s));
    gi += round_up((size_t)w->nnz[p] * 4, 256);
  }
  tern::B3Prep pr;
  std::memset(&pr, 0, sizeof(pr));
  pr.x = x;
  pr.x5 = const_cast<uint16_t*>(d.x5);
  pr.k = w->k;
  pr.m = m;
  pr.zero = d.rctr;  // the residual pass's counters start at zero (cleared in the launch: no memset node)
  pr.nzero = d.rctr ? b3_res_units(w) : 0;
  TERN_HIP(tern::launch_b3_prep(w->group, nullptr, 1, pr, w->k, s));
  const long nres = (long)b3_res_units(w) * d.rslots;
  if (d.rsum)
    TERN_HIP(tern::launch_b3_res(w->group, pick_mt(m), nullptr, nullptr, (int)nres, d, w->k,
                                 b3_res_lds_cap(nres, w->group, pick_mt(m), w->k),
                                 nullptr, 0, 0, s));
  const int items = d.row_blocks * parts;
  const int nwg = std::min(tern_cu_count(), (items + tern::kB3Waves - 1) / tern::kB3Waves);
  TERN_HIP(tern::launch_gemv_b3(w->group, pick_mt(m), nullptr, nullptr, nullptr, nwg, d, items, s));
  if (parts > 1) TERN_HIP(tern::launch_splitk_reduce(d.partial, parts, m, w->n, y, y_dtype == TERN_F32, s));
  return TERN_OK;
}

size_t tern_batch_workspace_bytes(const tern_matrix* w, int32_t count, int32_t m) {
  if (count <= 0 || m <= 0 || !w) return 0;
  if (gemm_route(m)) return gemm_batch_ws_bytes(w, count, m);
  if (b3_route_n(w, count, m)) {
    B3Batch b;
    return build_b3_batch(w, nullptr, nullptr, count, m, TERN_F16, nullptr, false, &b) == TERN_OK ? b.total : 0;
  }
  if (small_route(w[0].format, w[0].group, m)) return small_batch_ws_bytes(w, count, m);
  const int cmax = max_mt(w[0].format, w[0].group);
  const int mtp = pick_mt(std::min(m, cmax));
  std::vector<int> bns, bgps, bkw;
  batch_splits(w, count, m, mtp, &bns, &bgps, &bkw);
  size_t idx = 0;
  for (int i = 0; i < count; ++i) idx += index_bytes(&w[i]) + part_index_bytes(&w[i], bns[i]);
  const bool mf = use_mfma(w[0].format);
  // lane-per-row decode: one descriptor per work item, then the partials and
  // reduce table; matrix-core decode: two row ranges per (matrix, row
  // chunk), one record per workgroup (balanced placement may split items up
  // to the launch's resident slots: at most kMfmaMaxWgsPerCu per CU), then the
  // partials and reduce table (the layouts build_batch makes)
  // (arrival counters: one per row block of a descriptor with K parts; the
  // matrix-core placement cuts row blocks down to 16 rows at most)
  size_t nparts = 0, nitems = 0, coarse = 0, partial = 0, nctr = 0;
  for (int i = 0; i < count; ++i) {
    if (w[i].n <= 0 || w[i].k <= 0) continue;
    const int ns = bns[i];
    const int rpi = mf ? rows_per_item(bkw[i]) : tern::kGemvRows;
    const size_t rb = (size_t)(w[i].n + rpi - 1) / rpi;
    for (int c0 = 0; c0 < m; c0 += cmax) {
      const int mc = std::min(cmax, m - c0);
      ++nparts;
      nitems += rb * ns;
      coarse += rb * ns;
      if (ns > 1) {
        partial += round_up((size_t)ns * mc * w[i].n * 4, 256);
        nctr += mf ? (size_t)(w[i].n + tern::kGemvRows / 4 - 1) / (tern::kGemvRows / 4) : rb;
      }
    }
  }
  if (!mf) return round_up(nitems * sizeof(GemvDesc), 256) + round_up(partial + nctr * 4, 256) + idx;
  size_t recs_off, part_off;
  mfma_offsets(nparts, std::max(coarse, (size_t)tern_cu_count() * tern::kMfmaMaxWgsPerCu), &recs_off, &part_off);
  return round_up(part_off + partial + nctr * 4, 256) + idx;
}

tern_status tern_gemv_batched(const tern_matrix* w, const uint16_t* const* x, void* const* y,
                              int32_t count, int32_t m, int32_t y_dtype, void* ws, size_t ws_bytes,
                              void* stream) {
  std::vector<GemvDesc> items;
  int mt = 1, max_krp = 0;
  bool offsets = false;
  if (gemm_route(m)) {
    if (!ws) return fail(TERN_E_WORKSPACE, "batched product needs a workspace");
    TERN_TRY(check_dev(ws, true, "ws"));
    TileBatch b;
    TERN_TRY(build_gemm_batch(w, x, y, count, m, y_dtype, static_cast<char*>(ws), &b));
    if (b.tiles.empty()) return TERN_OK;
    const size_t need = tile_ws_bytes(b);
    if (ws_bytes < need) return fail(TERN_E_WORKSPACE, "batched product needs %zu workspace bytes", need);
    hipStream_t s = (hipStream_t)stream;
    char* base = static_cast<char*>(ws);
    const size_t tb = round_up(b.tiles.size() * sizeof(GemvDesc), 256);
    TERN_HIP(hipMemcpyAsync(base, b.tiles.data(), b.tiles.size() * sizeof(GemvDesc), hipMemcpyHostToDevice, s));
    if (!b.red.empty())
      TERN_HIP(hipMemcpyAsync(base + tb + b.partial_bytes, b.red.data(), b.red.size() * sizeof(tern::RedDesc),
                              hipMemcpyHostToDevice, s));
    TERN_HIP(tern::launch_gemm_grouped(reinterpret_cast<const GemvDesc*>(base), (int)b.tiles.size(), w[0].format,
                                       w[0].group, tern::gemm_tile_rows(m) / 64, b.np, b.offs, s));
    if (!b.red.empty())
      TERN_HIP(tern::launch_reduce_grouped(reinterpret_cast<const tern::RedDesc*>(base + tb + b.partial_bytes),
                                           (int)b.red.size(), b.red_blocks, s));
    return TERN_OK;
  }
  if (count > 0 && b3_route_n(w, count, m)) {
    B3Batch b;
    TERN_TRY(build_b3_batch(w, x, y, count, m, y_dtype, static_cast<char*>(ws), true, &b));
    if (b.descs.empty()) return TERN_OK;
    if (!ws || ws_bytes < b.total) return fail(TERN_E_WORKSPACE, "batched product needs %zu workspace bytes", b.total);
    TERN_TRY(check_dev(ws, true, "ws"));
    hipStream_t s = (hipStream_t)stream;
    TERN_TRY(upload_b3_batch(b, static_cast<char*>(ws), s, false));
    return run_b3_batch(b, w[0].group, static_cast<char*>(ws), s);
  }
  if (count > 0 && small_route(w[0].format, w[0].group, m)) {
    if (!ws) return fail(TERN_E_WORKSPACE, "batched product needs a workspace");
    TERN_TRY(check_dev(ws, true, "ws"));
    TileBatch b;
    TERN_TRY(build_small_batch(w, x, y, count, m, y_dtype, static_cast<char*>(ws), &b));
    if (b.tiles.empty()) return TERN_OK;
    const size_t need = tile_ws_bytes(b);
    if (ws_bytes < need) return fail(TERN_E_WORKSPACE, "batched product needs %zu workspace bytes", need);
    hipStream_t s = (hipStream_t)stream;
    char* base = static_cast<char*>(ws);
    const size_t tb = round_up(b.tiles.size() * sizeof(GemvDesc), 256);
    TERN_HIP(hipMemcpyAsync(base, b.tiles.data(), b.tiles.size() * sizeof(GemvDesc), hipMemcpyHostToDevice, s));
    if (!b.red.empty())
      TERN_HIP(hipMemcpyAsync(base + tb + b.partial_bytes, b.red.data(), b.red.size() * sizeof(tern::RedDesc),
                              hipMemcpyHostToDevice, s));
    TERN_HIP(tern::launch_gemm_small(reinterpret_cast<const GemvDesc*>(base), (int)b.tiles.size(), w[0].format,
                                     w[0].group, b.np, b.offs, s));
    if (!b.red.empty())
      TERN_HIP(tern::launch_reduce_grouped(reinterpret_cast<const tern::RedDesc*>(base + tb + b.partial_bytes),
                                           (int)b.red.size(), b.red_blocks, s));
    return TERN_OK;
  }
  std::vector<tern::WgRec> recs;
  DecodeSplits sp;
  TERN_TRY(build_batch(w, x, y, count, m, y_dtype, &items, &mt, &max_krp, &offsets, nullptr, &recs, &sp,
                       static_cast<char*>(ws)));
  if (items.empty()) return TERN_OK;
  // workspace: [descriptors][workgroup records (matrix-core decode)]
  // [partials of the K parts][arrival counters], at the offsets the builder
  // chose; the counters are cleared on the stream before the launch
  size_t need = std::max(items.size() * sizeof(GemvDesc), sp.ctr_off + sp.nctr * 4);
  if (!recs.empty()) need = std::max(need, sp.recs_off + recs.size() * sizeof(tern::WgRec));
  if (!ws || ws_bytes < need) return fail(TERN_E_WORKSPACE, "batched decode needs %zu workspace bytes", need);
  TERN_TRY(check_dev(ws, true, "ws"));
  hipStream_t s = (hipStream_t)stream;
  char* base = static_cast<char*>(ws);
  TERN_HIP(hipMemcpyAsync(base, items.data(), items.size() * sizeof(GemvDesc), hipMemcpyHostToDevice, s));
  if (!recs.empty())
    TERN_HIP(hipMemcpyAsync(base + sp.recs_off, recs.data(), recs.size() * sizeof(tern::WgRec), hipMemcpyHostToDevice, s));
  if (sp.nctr) TERN_HIP(hipMemsetAsync(base + sp.ctr_off, 0, sp.nctr * 4, s));
  const int nwg = recs.empty() ? (int)items.size() : (int)recs.size();
  TERN_HIP(launch_decode(w[0].format, w[0].group, mt, reinterpret_cast<const GemvDesc*>(base),
                         recs.empty() ? nullptr : reinterpret_cast<const tern::WgRec*>(base + sp.recs_off),
                         (int)items.size(), items[0], nwg, max_krp, offsets, s));
  return TERN_OK;
}

// A plan on the base-3 stream kernel (optionally with rotations folded into
// its activation preparation: rot[i] / xr[i] per product, or NULL).
static tern_status b3_plan_create(const tern_matrix* w, const uint16_t* const* x, void* const* y, int32_t count,
                                  int32_t m, int32_t y_dtype, void* ws, size_t ws_bytes,
                                  const uint16_t* const* rot, uint16_t* const* xr, int rot_block,
                                  tern_plan** out) {
  B3Batch b;
  TERN_TRY(build_b3_batch(w, x, y, count, m, y_dtype, static_cast<char*>(ws), true, &b, rot, xr, rot_block));
  char* base = static_cast<char*>(ws);
  if (!b.descs.empty()) {
    if (!ws || ws_bytes < b.total) return fail(TERN_E_WORKSPACE, "plan needs %zu workspace bytes", b.total);
    TERN_TRY(check_dev(ws, true, "ws"));
    TERN_TRY(upload_b3_batch(b, base, nullptr, true));
  }
  tern_plan* p = static_cast<tern_plan*>(std::malloc(sizeof(tern_plan)));
  if (!p) return fail(TERN_E_INVAL, "out of host memory");
  std::memset(p, 0, sizeof(*p));
  p->format = w[0].format;
  p->group = w[0].group;
  p->mt = b.mt;
  p->total_items = (int)b.items.size();
  p->b3 = true;
  p->dev = reinterpret_cast<const GemvDesc*>(base + b.descs_off);
  p->ndesc = (int)b.descs.size();
  p->preps = reinterpret_cast<const tern::B3Prep*>(base + b.preps_off);
  p->nprep = (int)b.preps.size();
  p->b3items = reinterpret_cast<const tern::B3Item*>(base + b.items_off);
  p->b3_maxk = b.max_k;
  p->b3res = reinterpret_cast<const tern::B3ResItem*>(base + b.res_off);
  p->nres = (int)b.res.size();
  p->queue = reinterpret_cast<uint32_t*>(base + b.queue_off);
  p->nwg = b.nwg;
  p->prep_first = b.prep_first;
  p->rot_block = rot_block;
  *out = p;
  return TERN_OK;
}

tern_status tern_plan_create(const tern_matrix* w, const uint16_t* const* x, void* const* y,
                             int32_t count, int32_t m, int32_t y_dtype, void* ws, size_t ws_bytes,
                             tern_plan** out) {
  if (!out) return fail(TERN_E_INVAL, "out is NULL");
  *out = nullptr;
  std::vector<GemvDesc> items;
  std::vector<int> mat;
  int mt = 1, max_krp = 0;
  bool offsets = false;
  if (gemm_route(m)) {
    TileBatch b;
    TERN_TRY(build_gemm_batch(w, x, y, count, m, y_dtype, static_cast<char*>(ws), &b));
    const size_t need = tile_ws_bytes(b);
    const size_t tb = round_up(b.tiles.size() * sizeof(GemvDesc), 256);
    char* base = static_cast<char*>(ws);
    if (!b.tiles.empty()) {
      if (!ws || ws_bytes < need) return fail(TERN_E_WORKSPACE, "plan needs %zu workspace bytes", need);
      TERN_TRY(check_dev(ws, true, "ws"));
      TERN_HIP(hipMemcpy(base, b.tiles.data(), b.tiles.size() * sizeof(GemvDesc), hipMemcpyHostToDevice));
      if (!b.red.empty())
        TERN_HIP(hipMemcpy(base + tb + b.partial_bytes, b.red.data(), b.red.size() * sizeof(tern::RedDesc),
                           hipMemcpyHostToDevice));
    }
    tern_plan* p = static_cast<tern_plan*>(std::malloc(sizeof(tern_plan)));
    if (!p) return fail(TERN_E_INVAL, "out of host memory");
  std::memset(p, 0, sizeof(*p));
    p->dev = reinterpret_cast<const GemvDesc*>(base);
    p->recs = nullptr;
    p->ndesc = (int)b.tiles.size();
    p->total_items = (int)b.tiles.size();
    p->format = count > 0 ? w[0].format : 0;
    p->group = count > 0 ? w[0].group : 128;
    p->mt = 0;
    p->max_krp = 0;
    p->offsets = false;
    p->gemm = true;
    p->small = false;
    p->aw = tern::gemm_tile_rows(m) / 64;
    p->np = b.np;
    p->offs = b.offs;
    p->red = b.red.empty() ? nullptr : reinterpret_cast<const tern::RedDesc*>(base + tb + b.partial_bytes);
    p->nred = (int)b.red.size();
    p->red_blocks = b.red_blocks;
    *out = p;
    return TERN_OK;
  }
  if (count > 0 && b3_route_n(w, count, m))
    return b3_plan_create(w, x, y, count, m, y_dtype, ws, ws_bytes, nullptr, nullptr, 0, out);
  if (count > 0 && small_route(w[0].format, w[0].group, m)) {
    if (!ws) return fail(TERN_E_WORKSPACE, "plan needs a workspace");
    TERN_TRY(check_dev(ws, true, "ws"));
    TileBatch b;
    TERN_TRY(build_small_batch(w, x, y, count, m, y_dtype, static_cast<char*>(ws), &b));
    const size_t need = tile_ws_bytes(b);
    if (!b.tiles.empty() && ws_bytes < need) return fail(TERN_E_WORKSPACE, "plan needs %zu workspace bytes", need);
    char* base = static_cast<char*>(ws);
    const size_t tb = round_up(b.tiles.size() * sizeof(GemvDesc), 256);
    if (!b.tiles.empty()) {
      TERN_HIP(hipMemcpy(base, b.tiles.data(), b.tiles.size() * sizeof(GemvDesc), hipMemcpyHostToDevice));
      if (!b.red.empty())
        TERN_HIP(hipMemcpy(base + tb + b.partial_bytes, b.red.data(), b.red.size() * sizeof(tern::RedDesc),
                           hipMemcpyHostToDevice));
    }
    tern_plan* p = static_cast<tern_plan*>(std::malloc(sizeof(tern_plan)));
    if (!p) return fail(TERN_E_INVAL, "out of host memory");
  std::memset(p, 0, sizeof(*p));
    p->dev = reinterpret_cast<const GemvDesc*>(base);
    p->recs = nullptr;
    p->ndesc = (int)b.tiles.size();
    p->total_items = (int)b.tiles.size();
    p->format = w[0].format;
    p->group = w[0].group;
    p->mt = 0;
    p->max_krp = 0;
    p->offsets = false;
    p->gemm = false;
    p->small = true;
    p->aw = 0;
    p->np = b.np;
    p->offs = b.offs;
    p->red = b.red.empty() ? nullptr : reinterpret_cast<const tern::RedDesc*>(base + tb + b.partial_bytes);
    p->nred = (int)b.red.size();
    p->red_blocks = b.red_blocks;
    *out = p;
    return TERN_OK;
  }
  std::vector<tern::WgRec> recs;
  DecodeSplits sp;
  TERN_TRY(build_batch(w, x, y, count, m, y_dtype, &items, &mt, &max_krp, &offsets, &mat, &recs, &sp,
                       static_cast<char*>(ws)));
  // workspace: [descriptors][workgroup records (matrix-core decode)]
  // [partials of the K parts][arrival counters][residual index of each
  // matrix], at the offsets the builder chose; the counters are cleared
  // here and every launch leaves them clear
  size_t tables = std::max(items.size() * sizeof(GemvDesc), sp.ctr_off + sp.nctr * 4);
  if (!recs.empty()) tables = std::max(tables, sp.recs_off + recs.size() * sizeof(tern::WgRec));
  tables = round_up(tables, 256);
  char* base = static_cast<char*>(ws);
  if (!items.empty()) {
    // K parts of each product (all of its descriptors share them)
    std::vector<int> parts(count, 1), pgps(count, 0);
    for (size_t t = 0; t < items.size(); ++t) {
      parts[mat[t]] = items[t].splits;
      pgps[mat[t]] = items[t].gps;
    }
    std::vector<size_t> ioff(count, 0), poff(count, 0);
    size_t need = tables;
    for (int i = 0; i < count; ++i) {
      ioff[i] = need;
      need += index_bytes(&w[i]);
      poff[i] = need;
      need += recs.empty() ? 0 : part_index_bytes(&w[i], parts[i]);
    }
    if (!ws || ws_bytes < need) return fail(TERN_E_WORKSPACE, "plan needs %zu workspace bytes", need);
    TERN_TRY(check_dev(ws, true, "ws"));
    // the residual indexes serve the matrix-core decode launch (records)
    auto part_ptrs = [&](int i, uint32_t** prow, uint8_t** pblk, uint32_t** pix) {
      char* q = base + poff[i];
      *prow = reinterpret_cast<uint32_t*>(q);
      q += round_up(((size_t)parts[i] * w[i].n + 1) * 4, 256);
      *pblk = reinterpret_cast<uint8_t*>(q);
      q += round_up(part_entries(&w[i]) * (w[i].group / 4), 256);
      *pix = reinterpret_cast<uint32_t*>(q);
    };
    if (!recs.empty())
      for (size_t t = 0; t < items.size(); ++t) {
        const int i = mat[t];
        if (plan_part_indexes(&w[i], parts[i])) {
          uint32_t *prow, *pix;
          uint8_t* pblk;
          part_ptrs(i, &prow, &pblk, &pix);
          items[t].prowptr = prow;
          items[t].pblocks = pblk;
          items[t].pidx = pix;
          items[t].pnnz = (uint32_t)part_entries(&w[i]);
        } else if (plan_indexes(&w[i])) {
          items[t].gidx[0] = reinterpret_cast<const uint32_t*>(base + ioff[i]);
        }
      }
    TERN_HIP(hipMemcpy(base, items.data(), items.size() * sizeof(GemvDesc), hipMemcpyHostToDevice));
    if (sp.nctr) TERN_HIP(hipMemset(base + sp.ctr_off, 0, sp.nctr * 4));
    if (!recs.empty()) {
      TERN_HIP(hipMemcpy(base + sp.recs_off, recs.data(), recs.size() * sizeof(tern::WgRec), hipMemcpyHostToDevice));
      for (int i = 0; i < count; ++i) {
        if (plan_part_indexes(&w[i], parts[i])) {
          uint32_t *prow, *pix;
          uint8_t* pblk;
          part_ptrs(i, &prow, &pblk, &pix);
          const uint32_t* msk[2] = {w[i].mask[0], w[i].mask[1]};
          const uint32_t* rpt[2] = {w[i].rowptr[0], w[i].rowptr[1]};
          const uint8_t* blk[2] = {w[i].blocks[0], w[i].blocks[1]};
          const uint16_t* rsc[2] = {w[i].rscale[0], w[i].rscale[1]};
          TERN_HIP(tern::launch_part_index(msk, rpt, blk, rsc, w[i].planes - 1, w[i].n, w[i].k / w[i].group,
                                           mask_words(w[i].k, w[i].group), w[i].group, parts[i], pgps[i], prow, pblk,
                                           pix, nullptr));
        } else if (plan_indexes(&w[i])) {
          TERN_HIP(tern::launch_res_index(w[i].mask[0], w[i].rowptr[0], w[i].rscale[0], w[i].n,
                                          mask_words(w[i].k, w[i].group),
                                          reinterpret_cast<uint32_t*>(base + ioff[i]), nullptr));
        }
      }
      TERN_HIP(tern::launch_tile_bounds(reinterpret_cast<const GemvDesc*>(base),
                                        reinterpret_cast<tern::WgRec*>(base + sp.recs_off), (int)recs.size(), nullptr));
    }
    // the index kernels ran on the null stream; wait for them only
    TERN_HIP(hipStreamSynchronize(nullptr));
  }
  tern_plan* p = static_cast<tern_plan*>(std::malloc(sizeof(tern_plan)));
  if (!p) return fail(TERN_E_INVAL, "out of host memory");
  std::memset(p, 0, sizeof(*p));
  p->dev = reinterpret_cast<const GemvDesc*>(base);
  p->recs = recs.empty() ? nullptr : reinterpret_cast<const tern::WgRec*>(base + sp.recs_off);
  p->ndesc = (int)items.size();
  p->total_items = recs.empty() ? (int)items.size() : (int)recs.size();
  p->format = count > 0 ? w[0].format : 0;
  p->group = count > 0 ? w[0].group : 128;
  p->mt = mt;
  p->max_krp = max_krp;
  p->offsets = offsets;
  p->gemm = false;
  p->small = false;
  p->aw = p->np = 0;
  p->red = nullptr;  // K parts are summed inside the decode launch
  p->nred = 0;
  p->red_blocks = 0;
  *out = p;
  return TERN_OK;
}

static tern_status plan_launch(const tern_plan* plan, hipStream_t s, hipEvent_t before, hipEvent_t after) {
  if (!plan) return fail(TERN_E_INVAL, "plan is NULL");
  for (int r = 0; r < plan->nrots; ++r) TERN_HIP(tern::launch_rotate(plan->rots[r], plan->rot_block, s));
  if (plan->b3 && plan->total_items > 0) {
    tern::B3Prep none;
    std::memset(&none, 0, sizeof(none));
    GemvDesc dummy;
    std::memset(&dummy, 0, sizeof(dummy));
    if (plan->nres == 0 || plan->prep_first) {
      // rotating preparations write what the residual pass reads: a launch of their own
      if (plan->prep_first)
        TERN_HIP(tern::launch_b3_prep_rot(plan->group, plan->rot_block, plan->preps, plan->nprep, plan->b3_maxk, s));
      else
        TERN_HIP(tern::launch_b3_prep(plan->group, plan->preps, plan->nprep, none, plan->b3_maxk, s));
      TERN_HIP(tern::launch_b3_res(plan->group, plan->mt, plan->dev, plan->b3res, plan->nres, dummy, plan->b3_maxk,
                                   b3_res_lds_cap(plan->nres, plan->group, plan->mt, plan->b3_maxk), nullptr, 0, 0, s));
    } else {  // the preparations ride along in the residual pass's launch
      TERN_HIP(tern::launch_b3_res(plan->group, plan->mt, plan->dev, plan->b3res, plan->nres, dummy, plan->b3_maxk,
                                   b3_res_lds_cap(plan->nres, plan->group, plan->mt, plan->b3_maxk), plan->preps, plan->nprep, plan->b3_maxk, s));
    }
    if (before) TERN_HIP(hipEventRecord(before, s));
    TERN_HIP(tern::launch_gemv_b3(plan->group, plan->mt, plan->dev, plan->b3items, plan->queue, plan->nwg, dummy,
                                  plan->total_items, s));
    if (after) TERN_HIP(hipEventRecord(after, s));
    return TERN_OK;
  }
  if (before) TERN_HIP(hipEventRecord(before, s));
  if (plan->total_items == 0) {
  } else if (plan->gemm) {
    TERN_HIP(tern::launch_gemm_grouped(plan->dev, plan->total_items, plan->format, plan->group, plan->aw, plan->np,
                                       plan->offs, s));
    if (plan->nred) TERN_HIP(tern::launch_reduce_grouped(plan->red, plan->nred, plan->red_blocks, s));
  } else if (plan->small) {
    TERN_HIP(tern::launch_gemm_small(plan->dev, plan->total_items, plan->format, plan->group, plan->np, plan->offs, s));
    if (plan->nred) TERN_HIP(tern::launch_reduce_grouped(plan->red, plan->nred, plan->red_blocks, s));
  } else if (plan->folded) {
    TERN_HIP(tern::launch_gemv_mfma_rot(plan->group, plan->mt, plan->dev, plan->recs, plan->ndesc, plan->total_items,
                                        plan->max_krp, plan->offsets, plan->fold, s));
    if (plan->nred) TERN_HIP(tern::launch_reduce_grouped(plan->red, plan->nred, plan->red_blocks, s));
  } else {
    GemvDesc dummy;
    std::memset(&dummy, 0, sizeof(dummy));
    TERN_HIP(launch_decode(plan->format, plan->group, plan->mt, plan->dev, plan->recs, plan->ndesc, dummy,
                           plan->total_items, plan->max_krp, plan->offsets, s));
    if (plan->nred) TERN_HIP(tern::launch_reduce_grouped(plan->red, plan->nred, plan->red_blocks, s));
  }
  if (after) TERN_HIP(hipEventRecord(after, s));
  return TERN_OK;
}

int64_t tern_b3_min_stages(int64_t stages) {
  const int64_t before = b3_min_stages();
  if (stages >= 0) g_b3_min_stages = stages;
  else if (stages == -1) g_b3_min_stages = -1;
  return before;
}

tern_status tern_plan_run(const tern_plan* plan, void* stream) {
  return plan_launch(plan, (hipStream_t)stream, nullptr, nullptr);
}

tern_status tern_plan_run_events(const tern_plan* plan, void* stream, void* before, void* after) {
  return plan_launch(plan, (hipStream_t)stream, (hipEvent_t)before, (hipEvent_t)after);
}

int32_t tern_plan_launches(const tern_plan* plan) {
  if (!plan) return -1;
  int32_t n = plan->nrots;
  if (plan->total_items == 0) return n;
  if (plan->b3) {
    const bool own_prep = plan->nres == 0 || plan->prep_first;
    return n + (own_prep && plan->nprep > 0 ? 1 : 0) + (plan->nres > 0 ? 1 : 0) + (plan->nwg > 0 ? 1 : 0);
  }
  return n + 1 + (plan->nred > 0 ? 1 : 0);
}

void tern_plan_destroy(tern_plan* plan) {
  if (plan) std::free(plan->rots);
  std::free(plan);
}

// A rotated plan's workspace: the counters of a folded rotation
// (tern::kRotSyncBytes), one rotated copy per distinct x, then the plan's
// own tables.
using tern::kRotSyncBytes;

size_t tern_rotated_workspace_bytes(const tern_matrix* w, int32_t count, int32_t m) {
  if (count <= 0 || m <= 0 || !w) return 0;
  size_t bytes = tern_batch_workspace_bytes(w, count, m) + kRotSyncBytes;
  for (int i = 0; i < count; ++i)
    if (w[i].k > 0) bytes += round_up((size_t)2 * m * w[i].k, 256);  // a rotated copy per product at most
  return bytes;
}

tern_status tern_plan_create_rotated(const tern_matrix* w, const uint16_t* const* x, const uint16_t* const* rot,
                                     int32_t rot_block, void* const* y, int32_t count, int32_t m, int32_t y_dtype,
                                     void* ws, size_t ws_bytes, tern_plan** out) {
  if (!out) return fail(TERN_E_INVAL, "out is NULL");
  *out = nullptr;
  if (!rot) return tern_plan_create(w, x, y, count, m, y_dtype, ws, ws_bytes, out);
  if (rot_block != 64 && rot_block != 128) return fail(TERN_E_UNSUPPORTED, "rotation blocks of 64 or 128 (got %d)", rot_block);
  if (count < 0 || m < 0) return fail(TERN_E_INVAL, "count=%d, m=%d must not be negative", count, m);
  if (count > 0 && (!w || !x || !y)) return fail(TERN_E_INVAL, "NULL descriptor, activation or output arrays");
  // the fold's counters, then one rotated copy per distinct (x, R), then the
  // plan's own workspace
  std::map<const uint16_t*, std::pair<const uint16_t*, size_t>> seen;  // x -> (R, offset of its copy)
  std::vector<const uint16_t*> xin(count > 0 ? count : 1);
  std::vector<uint16_t*> xr(count > 0 ? count : 1, nullptr);
  size_t off = kRotSyncBytes;
  for (int i = 0; i < count; ++i) {
    xin[i] = x[i];
    if (!rot[i] || w[i].n <= 0 || w[i].k <= 0 || m == 0) continue;
    if (w[i].k % rot_block) return fail(TERN_E_UNSUPPORTED, "product %d: k=%d is not a multiple of the rotation block", i, w[i].k);
    TERN_TRY(check_dev(rot[i], true, "rotation", 16));
    TERN_TRY(check_dev(x[i], true, "x", 16));
    auto it = seen.find(x[i]);
    if (it == seen.end()) {
      it = seen.insert({x[i], {rot[i], off}}).first;
      off += round_up((size_t)2 * m * w[i].k, 256);
    } else if (it->second.first != rot[i]) {
      return fail(TERN_E_INVAL, "product %d reads an x that another product rotates differently", i);
    }
    if (!ws) return fail(TERN_E_WORKSPACE, "a rotated plan needs a workspace");
    xr[i] = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + it->second.second);
    xin[i] = xr[i];
  }
  if (off > ws_bytes) return fail(TERN_E_WORKSPACE, "rotated plan needs more workspace");
  char* inner = static_cast<char*>(ws) + off;
  const size_t inner_bytes = ws_bytes - off;
  if (count > 0 && b3_route_n(w, count, m))  // folded into the activation preparation
    return b3_plan_create(w, x, y, count, m, y_dtype, inner, inner_bytes, rot, xr.data(), rot_block, out);
  TERN_TRY(tern_plan_create(w, xin.data(), y, count, m, y_dtype, inner, inner_bytes, out));
  // other routes: rotation launches (up to kMaxRotations inputs each) into the copies
  std::vector<tern::RotBatch> rb;
  std::map<const uint16_t*, bool> done;
  for (int i = 0; i < count; ++i) {
    if (!xr[i] || done[x[i]]) continue;
    done[x[i]] = true;
    if (rb.empty() || rb.back().count == tern::kMaxRotations) {
      tern::RotBatch a;
      std::memset(&a, 0, sizeof(a));
      a.m = m;
      rb.push_back(a);
    }
    tern::RotBatch& a = rb.back();
    a.R[a.count] = rot[i];
    a.x[a.count] = x[i];
    a.out[a.count] = xr[i];
    a.k[a.count] = w[i].k;
    a.begin[a.count + 1] = a.begin[a.count] + w[i].k / rot_block;
    ++a.count;
  }
  tern_plan* p = *out;
  // the matrix-core decode takes up to kMaxRotations inputs inside its own
  // launch: the shares first, then the product's workgroups
  if (rb.size() == 1 && !p->gemm && !p->small && !p->b3 && p->recs && p->total_items > 0 && use_mfma(p->format) &&
      m <= p->mt) {
    tern::RotFold& f = p->fold;
    f.a = rb[0];
    for (int i = 0; i <= f.a.count; ++i) f.a.begin[i] = 0;
    for (int i = 0; i < f.a.count; ++i)
      f.a.begin[i + 1] = f.a.begin[i] + (f.a.k[i] + tern::kRotShareRows - 1) / tern::kRotShareRows;
    f.block = rot_block;
    f.shares = f.a.begin[f.a.count];
    f.sync = static_cast<uint32_t*>(ws);
    hipError_t e = hipMemset(ws, 0, kRotSyncBytes);
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess) {
      tern_plan_destroy(p);
      *out = nullptr;
      return fail(TERN_E_HIP, "hipMemset: %s", hipGetErrorString(e));
    }
    p->folded = true;
    return TERN_OK;
  }
  if (!rb.empty()) {
    (*out)->rots = static_cast<tern::RotBatch*>(std::malloc(rb.size() * sizeof(tern::RotBatch)));
    if (!(*out)->rots) {
      tern_plan_destroy(*out);
      *out = nullptr;
      return fail(TERN_E_INVAL, "out of host memory");
    }
    std::memcpy((*out)->rots, rb.data(), rb.size() * sizeof(tern::RotBatch));
    (*out)->nrots = (int)rb.size();
    (*out)->rot_block = rot_block;
  }
  return TERN_OK;
}

tern_status tern_quantize(const uint16_t* w, int32_t n, int32_t k, int32_t group, const uint32_t* mask,
                          int32_t iters, int8_t* trits, uint16_t* scales, uint16_t* offset, void* stream) {
  if (n < 0 || k < 0) return fail(TERN_E_INVAL, "n=%d, k=%d must not be negative", n, k);
  if (group != 64 && group != 128) return fail(TERN_E_UNSUPPORTED, "quantize takes group 64 or 128 (got %d)", group);
  if (k % group) return fail(TERN_E_UNSUPPORTED, "k=%d must be a multiple of group %d", k, group);
  if (iters < 0 || iters > 1000) return fail(TERN_E_INVAL, "iters=%d must be in [0, 1000]", iters);
  if ((long long)n * k > (long long)INT32_MAX * 16) return fail(TERN_E_UNSUPPORTED, "matrix too large");
  if (n == 0 || k == 0) return TERN_OK;
  TERN_TRY(check_dev(w, true, "w", 2));
  TERN_TRY(check_dev(trits, true, "trits", 1));
  TERN_TRY(check_dev(scales, true, "scales", 2));
  TERN_TRY(check_dev(offset, true, "offset", 2));
  if (mask) TERN_TRY(check_dev(mask, true, "mask", 4));
  TERN_HIP(tern::launch_quantize(w, n, k, group, mask, mask_words(k, group), iters, trits, scales, offset,
                                 (hipStream_t)stream));
  return TERN_OK;
}

tern_status tern_rotate_batched(int32_t count, const uint16_t* const* R, int32_t block, const uint16_t* const* x,
                                const int32_t* k, int32_t m, uint16_t* const* out, void* stream) {
  if (count < 0 || count > tern::kMaxRotations)
    return fail(TERN_E_UNSUPPORTED, "count=%d: one launch rotates 0..%d inputs", count, tern::kMaxRotations);
  if (m < 0) return fail(TERN_E_INVAL, "m=%d must not be negative", m);
  if (block != 64 && block != 128) return fail(TERN_E_UNSUPPORTED, "rotate takes block 64 or 128 (got %d)", block);
  if (count > 0 && (!R || !x || !k || !out)) return fail(TERN_E_INVAL, "NULL argument arrays");
  tern::RotBatch a;
  std::memset(&a, 0, sizeof(a));
  a.m = m;
  int blocks = 0;
  for (int i = 0; i < count; ++i) {
    if (k[i] < 0) return fail(TERN_E_INVAL, "k[%d]=%d must not be negative", i, k[i]);
    if (k[i] % block) return fail(TERN_E_UNSUPPORTED, "k[%d]=%d must be a multiple of block %d", i, k[i], block);
  }
  if (m == 0) return TERN_OK;
  for (int i = 0; i < count; ++i) {
    if (k[i] == 0) continue;
    TERN_TRY(check_dev(R[i], true, "R", 16));
    TERN_TRY(check_dev(x[i], true, "x", 4));
    TERN_TRY(check_dev(out[i], true, "out", 4));
    a.R[a.count] = R[i];
    a.x[a.count] = x[i];
    a.out[a.count] = out[i];
    a.k[a.count] = k[i];
    a.begin[a.count] = blocks;
    blocks += k[i] / block;
    ++a.count;
  }
  a.begin[a.count] = blocks;
  if (a.count == 0) return TERN_OK;
  TERN_HIP(tern::launch_rotate(a, block, (hipStream_t)stream));
  return TERN_OK;
}

tern_status tern_rotate(const uint16_t* R, int32_t block, const uint16_t* x, int32_t m, int32_t k, uint16_t* out,
                        void* stream) {
  if (m < 0 || k < 0) return fail(TERN_E_INVAL, "m=%d, k=%d must not be negative", m, k);
  uint16_t* o = out;
  return tern_rotate_batched(1, &R, block, &x, &k, m, &o, stream);
}

tern_status tern_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes % 16) return fail(TERN_E_INVAL, "bytes=%zu is not a multiple of 16", bytes);
  if (bytes == 0) return TERN_OK;
  TERN_TRY(check_dev(buf, true, "buf"));
  TERN_TRY(check_dev(sink, true, "sink", 4));
  TERN_HIP(tern::launch_read_probe(buf, bytes, sink, (hipStream_t)stream));
  return TERN_OK;
}

tern_status tern_bits(const tern_matrix* w, double* info, double* plane, double* storage) {
  if (!w) return fail(TERN_E_INVAL, "matrix descriptor is NULL");
  TERN_TRY(check_shape(w->n, w->k, w->group, w->planes, w->format, w->offset_mode));
  const double weights = (double)w->n * (double)w->k;
  if (weights == 0) return fail(TERN_E_INVAL, "empty matrix");
  size_t sz[TERN_NBUF];
  TERN_TRY(tern_packed_sizes(w->n, w->k, w->group, w->format, w->planes, w->nnz, w->offset_mode, sz));
  double trits = weights, planeb = (double)sz[TERN_BUF_PLANE0], total = 0;
  for (int p = 0; p < w->planes - 1; ++p) {
    trits += (double)w->nnz[p] * w->group;
    planeb += (double)sz[TERN_BUF_BLOCKS1 + p];
  }
  for (int i = 0; i < TERN_NBUF; ++i) total += (double)sz[i];
  if (w->planes > 1) total += (double)(w->planes - 2) * (sz[TERN_BUF_MASK] + sz[TERN_BUF_ROWPTR]);
  if (info) *info = std::log2(3.0) * trits / weights;
  if (plane) *plane = 8.0 * planeb / weights;
  if (storage) *storage = 8.0 * total / weights;
  return TERN_OK;
}

const char* tern_status_str(tern_status s) {
  switch (s) {
    case TERN_OK: return "TERN_OK";
    case TERN_E_INVAL: return "TERN_E_INVAL";
    case TERN_E_ALIGN: return "TERN_E_ALIGN";
    case TERN_E_UNSUPPORTED: return "TERN_E_UNSUPPORTED";
    case TERN_E_CORRUPT: return "TERN_E_CORRUPT";
    case TERN_E_WORKSPACE: return "TERN_E_WORKSPACE";
    case TERN_E_HIP: return "TERN_E_HIP";
  }
  return "TERN_E_UNKNOWN";
}

const char* tern_last_error(void) { return g_err; }

}  // extern "C"
