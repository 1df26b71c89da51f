// Internal declarations shared by the host API (tern_api.cpp) and the HIP
// kernel sources.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tern {

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

// Plain streaming read of bytes (a multiple of 16) from buf (measurement).
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

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
// descriptor with the most (0..2).
hipError_t launch_gemm_grouped(const GemvDesc* descs, int count, int format, int group, int aw, int np,
                               hipStream_t stream);
// Small-M (m <= 16) matrix-core product, grouped: one descriptor per
// workgroup, a 16 x 128 tile at column tn0 over K steps [tm0, splits) of 64;
// partial slice gps >= 0 writes FP32 sums to partial[gps][m][n], gps < 0
// writes y.  np as above.
hipError_t launch_gemm_small(const GemvDesc* descs, int count, int format, int group, int np, hipStream_t stream);
// Split sums of a grouped small-M launch: product i's blocks start at
// rd[i].begin (ascending), 256 outputs per block.
struct RedDesc {
  const float* partial;  // [splits][m][n]
  void* y;               // [m][n]
  int32_t splits, m, n, y_f32;
  int32_t begin;         // first block of this product
};
hipError_t launch_reduce_grouped(const RedDesc* rd, int count, int blocks, hipStream_t stream);

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
