// Internal declarations shared by the host API (tern_api.cpp) and the HIP
// kernel sources.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tern.h"

namespace tern {

// Records msg as the calling thread's last error (tern_last_error) and
// returns s (host code).
tern_status record_failure(tern_status s, const char* msg);

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kGemvRows = 64;      // rows per decode work item: one row per lane
constexpr int kMaxMT = 8;          // activation rows per decode pass

// Device-side description of one product (one matrix, one activation block).
struct GemvDesc {
  const uint8_t* plane0;
  const uint16_t* scale0;
  const uint32_t* mask[2];
  const uint32_t* rowptr[2];
  const uint8_t* blocks[2];
  const uint16_t* rscale[2];
  uint32_t nnz[2];        // residual entries of planes 1 and 2
  const uint16_t* offset;
  const uint16_t* x;      // [m][k]
  void* y;                // [m][n]
  float* partial;         // [splits][m][n] fp32 when splits > 1
  int32_t n, k, group, planes, offset_mode;
  int32_t m;              // activation rows handled by this descriptor (<= MT)
  int32_t stride;         // plane-0 row stride in bytes
  int32_t ng;             // groups per row
  int32_t mwords;         // mask words per row
  int32_t splits;         // K splits (work items along K)
  int32_t gps;            // groups per split
  int32_t row_blocks;     // work items along the rows: ceil(n / rows per item)
  int32_t tile_begin;     // first work-item index of this descriptor in the grid
  int32_t y_f32;          // 1: y is fp32, 0: fp16
  int32_t kwaves;         // matrix-core kernel: wavefronts sharing one 16-row tile's K (1, 2, 4)
  // Residual index prepared with a plan (matrix-core decode kernel; NULL
  // otherwise): per entry of the first residual plane, (group | FP16 scale
  // bits << 16); the entry ranges of the tiles are in the launch's records.
  const uint32_t* gidx[2];
  // Residual index per K part prepared with a plan (matrix-core decode
  // kernel, products cut into K parts or with two residual planes; NULL
  // otherwise): the entries of every residual plane ordered by (K part,
  // row, plane, group), with their blocks copied in that order (pblocks,
  // group/4 bytes each) and (group relative to the part | FP16 scale bits
  // << 16) in pidx; part s's row r starts at prowptr[s * n + r]
  // (prowptr[splits * n] = pnnz, the total).
  const uint32_t* pidx;
  const uint8_t* pblocks;
  const uint32_t* prowptr;
  uint32_t pnnz;
  // Grouped matrix-core product: origin of this workgroup's output tile.
  int32_t tm0, tn0;
  // Matrix-core decode kernel: first row of this descriptor's row range
  // (a matrix may be covered by two ranges with different kwaves).
  int32_t row_base;
  // Matrix-core tiles: K part [ks0, ks1) in 64-trit steps, and the FP32
  // partial slice it writes (kpart >= 0) instead of y.
  int32_t ks0, ks1, kpart;
  // Decode kernels with splits > 1: one arrival counter per row block of
  // this descriptor (zero before the launch; the launch leaves it zero), so
  // the last workgroup of a row block sums the K parts and writes y; NULL:
  // only the partials are written (a separate reduce sums them).
  uint32_t* ctr;
  // Base-3 matrix-core decode: the activations in its slot order
  // ([m][ng][b3_chunks_per_group][4] FP16) and, with an offset, the FP32
  // group sums of x ([m][ng]); both prepared by launch_b3_prep.  There,
  // the first p0 parts are K parts of plane 0 (gps 208-byte stages each)
  // and, when splits > p0, part p0 adds the residual planes and the offset
  // over the whole row; splits parts in all are summed in part order.
  const uint16_t* x5;
  const float* xs;
  int32_t p0;
  // Base-3 matrix-core decode: FP32 sums of the residual planes and the
  // offset per output ([m][n]), written by launch_b3_res before the product
  // and added to y by it; NULL when the matrix has neither.
  const float* rsum;
  // Residual pass: each residual plane's entries of a row block are cut into
  // rsplit ranges; rslots = max(1, (planes - 1) * rsplit) units per row
  // block (slot = plane * rsplit + range; slot 0 also adds the offset).
  // With rslots > 1 every unit stores its rows' sums in rpart
  // ([rslots][m][n] FP32) and the row block's last unit (arrival counter
  // rctr[row block], zero between launches) adds them in slot order into
  // rsum.
  int32_t rsplit, rslots;
  float* rpart;
  uint32_t* rctr;
};

// ---- decode products (gemv.hip)
// Launches the lane-per-row decode kernel over total_items work items: with
// ndesc > 0, descs (device memory) holds one descriptor per work item (the
// descriptor of the matrix the item belongs to, whose tile_begin is the
// matrix's first item); with ndesc == 0 every item uses `one`.  Descriptors
// with splits > 1 write FP32 partials; launch_splitk_reduce then sums them.
hipError_t launch_gemv(int format, int group, int mt, const GemvDesc* descs, int ndesc, const GemvDesc& one,
                       int total_items, hipStream_t stream);
// y[m][n] = sum_s partial[s][m][n] in split order.
hipError_t launch_splitk_reduce(const float* partial, int splits, int m, int n, void* y,
                                int y_f32, hipStream_t stream);
// Groups per LDS stage of the decode kernel; K splits start on multiples of it.
int gemv_stage_groups(int format, int group);

// ---- matrix-core decode product for 2-bit planes (gemv_mfma.hip)
// Activation rows per pass (8 for group 128, 4 for group 64) and the longest
// K range (trits) one work item stages, for `mp` padded activation rows.
int gemv_mfma_max_rows(int group);
int gemv_mfma_max_range(int mp);
// Workgroups of the matrix-core decode kernel that one CU holds at once
// (LDS and register limits) for a launch with these parameters.
// Most workgroups per CU that a matrix-core decode launch is placed for
// (the workspace layout reserves one record per such slot).
constexpr int kMfmaMaxWgsPerCu = 3;
int gemv_mfma_wgs_per_cu(int group, int mp, int max_krp, bool offsets);
// Same descriptors and work items as launch_gemv; a work item is 64 / kwaves
// rows; K splits start on 256-trit blocks.  max_krp = the longest range of
// any descriptor rounded up to 256; offsets = some descriptor has an offset.
// Per-workgroup record of a grouped matrix-core decode launch (32 bytes):
// ri = range descriptor index << 20 | work item within the range, and the
// first residual plane's entry index at each 16-row tile boundary of the
// item (filled by launch_tile_bounds when the range has a residual index).
struct WgRec {
  uint32_t ri;
  uint32_t te[5];
  uint32_t pad[2];
};
// Matrix-core decode launch over total_items workgroups: with ndesc > 0,
// descs (device memory) holds the launch's row-range descriptors and recs
// one record per workgroup; with ndesc == 0 every workgroup uses `one`
// (item = workgroup index).
hipError_t launch_gemv_mfma(int group, int mp, const GemvDesc* descs, const WgRec* recs, int ndesc, const GemvDesc& one,
                            int total_items, int max_krp, bool offsets, hipStream_t stream);

// Residual index of a plan: for row n's j-th masked group g, entry
// e = rowptr[n] + j gets gidx[e] = g | rscale[e] << 16 (one thread per row).
hipError_t launch_res_index(const uint32_t* mask, const uint32_t* rowptr, const uint16_t* rscale, int n,
                            int mwords, uint32_t* gidx, hipStream_t stream);
// For each of `count` workgroup records whose range descriptor has a
// residual index: te[t] = rowptr[0][min(row0 + 16 t, n)], t = 0..4, where
// row0 is the item's first row.
hipError_t launch_tile_bounds(const GemvDesc* ranges, WgRec* recs, int count, hipStream_t stream);
// Residual index per K part of one product (see GemvDesc::pidx): nres
// residual planes (1 or 2), K parts of gps groups.  Counts into prowptr,
// scans it, then fills pblocks and pidx (three launches).
hipError_t launch_part_index(const uint32_t* const* mask, const uint32_t* const* rowptr, const uint8_t* const* blocks,
                             const uint16_t* const* rscale, int nres, int n, int ng, int mwords, int group, int parts,
                             int gps, uint32_t* prowptr, uint8_t* pblocks, uint32_t* pidx, hipStream_t stream);

// Plain streaming read of bytes (a multiple of 16) from buf (measurement).
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// ---- base-3 matrix-core decode (gemv_b3.hip), up to 4 activation rows
constexpr int kB3Waves = 7;          // wavefronts per workgroup; one workgroup per CU (LDS)
// Work item of a grouped launch: descriptor index << 16 | K part, and the
// 64-row block.  The items are split into kB3Queues lists of about equal
// cost, one per XCD (workgroup b serves list b % kB3Queues), each in
// decreasing cost.  Queue q is the words [q * kB3QueueWords, + 4): the next
// item beyond the first (taken from a counter), the finished wavefronts
// (both zero between launches), and the list's first and end item.
constexpr int kB3Queues = 8;
constexpr int kB3QueueWords = 1024;  // 4 KB apart
struct B3Item {
  uint32_t dp;
  uint32_t rb;
};
// Activation preparation of one product: x [m][k] FP16 -> x5 (slot order)
// and, if xs is not NULL, FP32 group sums xs [m][k/group]; m <= 4.
struct B3Prep {
  const uint16_t* x;
  uint16_t* x5;
  float* xs;
  int32_t k, m;
  uint32_t* zero;  // if not NULL: nzero words cleared (counters of the passes that follow)
  int32_t nzero;
  // rotated plans (launch_b3_prep_rot): if R is not NULL, the activations
  // are rotated first, blockdiag(R) x with R fp16 [k/rblock][rblock][rblock]
  // (FP32 sums, FP16 values); x5 holds the rotated values and xr [m][k] a
  // copy of them in position order
  const uint16_t* R;
  uint16_t* xr;
  int32_t rblock;
};
// Instructions (4-slot chunks) per group: 33 at group 128, 16 at group 64;
// groups per 208-byte stage: 8 and 16.
int b3_chunks_per_group(int group);
int b3_stage_groups(int group);
// Residual pass work unit: descriptor index, block of kB3ResRows output
// rows and slot (see GemvDesc::rslots).  One workgroup per unit.
constexpr int kB3ResRows = 256;
struct B3ResItem {
  uint32_t desc;
  uint32_t rb;
  uint32_t slot;
  uint32_t a0, a1;  // the unit's entries (launch_b3_res_ranges)
};
// Fills a0 and a1 of every unit of a table from the row pointers (after the
// descriptors and units are in device memory; again whenever rowptr changes).
hipError_t launch_b3_res_ranges(const GemvDesc* descs, B3ResItem* units, int nunits, hipStream_t stream);
// nunits workgroups over units (device), or with units == NULL the units
// (row block * rslots + slot) of the single descriptor `one`.  max_k: the
// longest k; lds_cap: the most LDS bytes a workgroup may take (a large
// activation window for launches of few units, smaller ones for occupancy).
// With units, the nprep activation preparations in preps (device; longest
// k prep_max_k; none when preps is NULL) run in the same launch, as
// launch_b3_prep would (their zero fields must be NULL: the units do not
// wait for them).  Nothing is launched when nunits is 0.
// Whole groups of activations (of mt rows) in a residual-pass window whose
// workgroup takes at most lds_cap bytes of LDS, for a launch whose longest
// product has max_k inputs (every group when they fit).
int b3_res_window_groups(int group, int mt, int max_k, int lds_cap);
hipError_t launch_b3_res(int group, int mt, const GemvDesc* descs, const B3ResItem* units, int nunits,
                         const GemvDesc& one, int max_k, int lds_cap, const B3Prep* preps, int nprep,
                         int prep_max_k, hipStream_t stream);
// preps (device) holds count preparations; with preps == NULL, `one` alone;
// max_k: the longest k among them.
hipError_t launch_b3_prep(int group, const B3Prep* preps, int count, const B3Prep& one, int max_k, hipStream_t stream);
// The preparation of a rotated plan's count products (device table; block =
// the plan's rotation block, 64 or 128): rotates the products with R, copies
// the others, and clears every zero list; one launch.
hipError_t launch_b3_prep_rot(int group, int block, const B3Prep* preps, int count, int max_k, hipStream_t stream);
// nwg workgroups.  With descs (device), the items table and the queues
// (kB3Queues * kB3QueueWords device words; the launch leaves the counters
// zero) drive the wavefronts; with descs == NULL every wavefront w takes
// items w, w + W, ... (W = nwg * kB3Waves) below nitems of the single
// descriptor `one` (item = K part * row_blocks + row block).  mt: 1, 2 or 4
// rows per pass.  Launches that share queues must not overlap.
hipError_t launch_gemv_b3(int group, int mt, const GemvDesc* descs, const B3Item* items, uint32_t* queue, int nwg,
                          const GemvDesc& one, int nitems, hipStream_t stream);

// ---- MFMA product (gemm.hip)
hipError_t launch_gemm(const GemvDesc& d, int format, hipStream_t stream);
// Activation rows per matrix-core tile for m activation rows (256 or 128).
inline int gemm_tile_rows(int m) { return m > 128 ? 256 : 128; }
// Workgroups of the large-tile matrix-core kernel one CU holds (LDS limit).
int gemm_wgs_per_cu(int format, int aw);
// Grouped matrix-core product: descs (device memory) holds one descriptor per
// workgroup with its tile origin (tm0, tn0) and K steps [ks0, ks1) (ks0 a
// multiple of 4); kpart >= 0 writes FP32 sums to partial[kpart][m][n]
// instead of y; aw = gemm_tile_rows(m) / 64; np = residual planes of the
// descriptor with the most (0..2); offsets: some descriptor has an offset.
// np and offsets pick the decode's precision (gemm_wide).
hipError_t launch_gemm_grouped(const GemvDesc* descs, int count, int format, int group, int aw, int np,
                               bool offsets, hipStream_t stream);
// Small-M (m <= 16) matrix-core product, grouped: one descriptor per
// workgroup, a 16 x 128 tile at column tn0 over K steps [tm0, splits) of 64;
// partial slice gps >= 0 writes FP32 sums to partial[gps][m][n], gps < 0
// writes y.  np and offsets as above.
hipError_t launch_gemm_small(const GemvDesc* descs, int count, int format, int group, int np, bool offsets,
                             hipStream_t stream);
// Whether the tile decode forms W~ in FP32 and rounds it once (products
// whose FP16 multiply-add chain would round more than once: an offset with
// residual planes, or two residual planes) instead of FP16 multiply-adds.
bool gemm_wide(int np, bool offsets);
// Split sums of a grouped small-M launch: product i's blocks start at
// rd[i].begin (ascending), 256 outputs per block.
struct RedDesc {
  const float* partial;  // [splits][m][n]
  void* y;               // [m][n]
  int32_t splits, m, n, y_f32;
  int32_t begin;         // first block of this product
};
hipError_t launch_reduce_grouped(const RedDesc* rd, int count, int blocks, hipStream_t stream);

// One product's 16-row matrix-core tiles described compactly, for the tiles
// and reduce table to be written on the device (tern_gemv: no table comes
// from host memory, so the call can be captured).  Tile t is chunk t /
// (nsplit * ntn), split (t / ntn) % nsplit, columns 128 * (t % ntn): the
// chunk's base descriptor with tn0, tm0 = rg[split], splits = rg[split + 1]
// and gps = split (or -1 with one split).
constexpr int kSmallMaxRanges = 64;
struct SmallSpec {
  GemvDesc base[2];                   // per 16-row activation chunk
  RedDesc red[2];                     // the chunks' reduce entries (nsplit > 1)
  int32_t nchunk, nsplit, ntn, nred;
  int32_t rg[kSmallMaxRanges + 1];    // step ranges of the splits
};
hipError_t launch_small_tiles(const SmallSpec& spec, GemvDesc* tiles, RedDesc* red, hipStream_t stream);

// ---- quantizer front-end (quant.hip)
// w fp16 [n][k] -> trits int8 [2][n][k], scales fp16 [2][n][k/group],
// offsets fp16 [n][k/group]; mask: u32 bitmap [n][mwords] of the groups that
// get the second plane (NULL: none); group 64 or 128.
hipError_t launch_quantize(const uint16_t* w, int n, int k, int group, const uint32_t* mask, int mwords, int iters,
                           int8_t* trits, uint16_t* scales, uint16_t* offset, hipStream_t stream);

// ---- activation rotation (rotate.hip)
// out_i[m][k_i] = blockdiag(R_i) x_i for up to kMaxRotations inputs in one
// launch: R_i fp16 [k_i/block][block][block], block 64 or 128; begin[i] =
// first workgroup (block) of input i, begin[count] = total blocks.
constexpr int kMaxRotations = 8;
struct RotBatch {
  const uint16_t* R[kMaxRotations];
  const uint16_t* x[kMaxRotations];
  uint16_t* out[kMaxRotations];
  int32_t k[kMaxRotations];
  int32_t begin[kMaxRotations + 1];
  int32_t count, m;
};
hipError_t launch_rotate(const RotBatch& a, int block, hipStream_t stream);

// The rotation folded into a matrix-core decode launch (plans only).  The
// launch's first `shares` workgroups each rotate kRotShareRows consecutive
// positions of one input into a.out (a.begin counts shares: ceil(k_i /
// kRotShareRows) per input) with write-through stores and count themselves
// in; the last raises kRotFlags copies of a ready flag.  Every later
// workgroup requests its first weight blocks, waits for its group's flag
// copy, and then stages its activations (the descriptors' x, which point
// into a.out).  The counters clear themselves by the end of each launch
// (sync: kRotSyncBytes, zero before the first launch; layout in
// gemv_mfma.hip).  The wait is bounded; a wait that gives up sets word 2.
// Launches of one plan must not overlap.
constexpr int kRotShareRows = 128;
constexpr int kRotFlags = 64;
constexpr int kRotSubs = 16;       // share sub-counts (the shares' count-in has two levels)
constexpr int kRotLineWords = 64;  // 256 bytes
constexpr size_t kRotSyncBytes = (size_t)(kRotFlags + 1 + kRotSubs) * kRotLineWords * 4;
struct RotFold {
  RotBatch a;
  int32_t block, shares;
  uint32_t* sync;  // kRotSyncBytes, zero before the first launch
};
hipError_t launch_gemv_mfma_rot(int group, int mp, const GemvDesc* descs, const WgRec* recs, int ndesc,
                                int total_items, int max_krp, bool offsets, const RotFold& rot, hipStream_t stream);

// ---- packing (pack.hip)
hipError_t launch_pack_plane0(int format, const int8_t* trits, int n, int k, int group,
                              int stride, uint8_t* plane0, uint32_t* flag, hipStream_t stream);
hipError_t launch_unpack_plane0(int format, const uint8_t* plane0, int n, int k, int group,
                                int stride, int8_t* trits, uint32_t* flag, hipStream_t stream);
// rowptr[0] = 0, rowptr[r+1] = popcount(mask row r); flags bits past ng.
hipError_t launch_mask_counts(const uint32_t* mask, int n, int ng, int mwords, uint32_t* rowptr,
                              uint32_t* flag, hipStream_t stream);
// In-place inclusive scan of rowptr[1..n] (single workgroup).
hipError_t launch_rowptr_scan(uint32_t* rowptr, int n, hipStream_t stream);
hipError_t launch_pack_residual(const int8_t* trits_p, const uint16_t* rscale_dense,
                                const uint32_t* mask, const uint32_t* rowptr, int n, int k,
                                int group, int mwords, uint8_t* blocks, uint16_t* rscale,
                                uint32_t* flag, hipStream_t stream);
hipError_t launch_unpack_residual(const uint8_t* blocks, const uint32_t* mask,
                                  const uint32_t* rowptr, int n, int k, int group, int mwords,
                                  int8_t* trits_p, uint32_t* flag, hipStream_t stream);
// flag |= bit if a[i] != b[i] for some i < count.
hipError_t launch_compare_u32(const uint32_t* a, const uint32_t* b, int count, uint32_t bit,
                              uint32_t* flag, hipStream_t stream);

// Validation flag bits written by the packing kernels.
constexpr uint32_t kFlagBadTrit = 1u;        // trit outside {-1,0,1}
constexpr uint32_t kFlagOutsideMask = 2u;    // residual trit set outside its mask
constexpr uint32_t kFlagMaskBits = 4u;       // mask bit set past the last group
constexpr uint32_t kFlagBadCode = 8u;        // invalid 2-bit code / base-3 byte / pad trit
constexpr uint32_t kFlagRowptr = 16u;        // rowptr disagrees with the mask

}  // namespace tern
