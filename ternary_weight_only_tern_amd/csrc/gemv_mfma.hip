// Decode-path product y = x W^T for up to 8 activation rows on packed 2-bit
// ternary planes, with the multiply-adds on the matrix cores.  Direct ternary
// execution ("Can ternary LLMs hit 1.58 bits per weight", How It Works: the
// packed weights are consumed without materialising a dense copy; arXiv
// 2609.09240 on packed planes executed directly).
//
// Work split.  A workgroup of 4 wavefronts owns 64 output rows and one range
// of K; each wavefront owns 16 rows.  Lane (q = lane / 16, r = lane % 16)
// streams row r: for every 256-trit block of the range it loads the 16 bytes
// (64 trits) at block offset 16*q straight into registers, several blocks
// ahead.  Nothing of the weights goes through LDS.
//
// Decode.  A 2-bit word holds 16 trits, even offsets in the low half-word and
// odd offsets in the high half-word, each a two's-complement 2-bit code.
// Shifting pair i to bits 14..15 / 30..31 and masking with 0xC000C000 gives
// the FP16 pair (2*t[2i], 2*t[2i+1]) exactly (0x4000 = 2.0, 0xC000 = -2.0).
// Four such pair words are the B operand of one v_mfma_f32_16x16x32_f16
// (B[kappa][n] = 2*W[row n][k(kappa)]), so the VALU only decodes and the
// matrix cores do the products; the 0.5 is folded into the scale.
//
// Group slots.  The A operand has 16 rows but there are at most 8 activation
// rows.  Its rows are used as (activation row, group) slots: slot
// m*GW + g holds x_m restricted to group g of the current window of GW
// groups and zero elsewhere, so D[slot][n] accumulates the per-group partial
// sum of row n, exactly the quantity the group scale multiplies.  A lane
// whose slot is inactive for a block reads its A operand from a zero area in
// LDS; the activations of the range are staged in LDS once per workgroup.
// At the end of each window every lane scales its four D values by the
// matching FP16 scales and adds them to its FP32 row accumulator.
//
// Residual planes are sparse; their blocks are listed per wavefront
// (row-major, so every row's entries are contiguous) and processed 16 at a
// time: entry e is B column e and A row e (each A row holds the activations
// of its entry's own group), and the diagonal of D is the entry's partial
// sum.  Rows add their entries' scaled values in entry order.  Offsets use
// per-group activation sums computed once per workgroup.  All sums are in a
// fixed order, so results are bitwise reproducible.
#include <algorithm>

#include "internal.h"

#define GLOBAL __attribute__((address_space(1)))

namespace tern {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;          // wavefronts per workgroup
constexpr int kRowsWave = 16;      // output rows per wavefront (MFMA N)
constexpr int kBlockTrits = 256;   // trits per block: 4 lanes x 64 trits of one row
constexpr int kMaxBlocks = 12;     // blocks per wavefront (all in flight at once)
constexpr int kZeroBytes = 128;    // zero A operands for inactive slots
constexpr int kResCap = 64;        // residual entries listed per pass and wavefront
constexpr int kResStage = 256;     // residual entries a workgroup stages in LDS (plan index)

template <typename T>
__device__ __forceinline__ const GLOBAL T* gp(const T* p) { return (const GLOBAL T*)p; }

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// B operands of the four MFMAs fed by two 2-bit words w0, w1 (32 trits):
// b[0] = pairs 0..3 of w0, b[1] = pairs 4..7 of w0, b[2], b[3] likewise of w1.
// One 64-bit shift serves both words: the high word picks up bits of w0 only
// below bit 14, which the mask clears.
__device__ __forceinline__ void decode_two(uint32_t w0, uint32_t w1, h8_t* b) {
  const uint64_t wd = ((uint64_t)w1 << 32) | w0;
  u4_t lo[2], hi[2];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint64_t s = wd << (14 - 2 * p);
    lo[p / 4][p % 4] = (uint32_t)s & 0xC000C000u;
    hi[p / 4][p % 4] = (uint32_t)(s >> 32) & 0xC000C000u;
  }
  b[0] = __builtin_bit_cast(h8_t, lo[0]);
  b[1] = __builtin_bit_cast(h8_t, lo[1]);
  b[2] = __builtin_bit_cast(h8_t, hi[0]);
  b[3] = __builtin_bit_cast(h8_t, hi[1]);
}

__device__ __forceinline__ h8_t lds_h8(const uint8_t* lds, uint32_t off) {
  return *reinterpret_cast<const h8_t*>(lds + off);
}

// 16 bytes (64 trits) of block c of the row at `wrow`; reads past the range
// are clamped onto its last 16 bytes (their activations are zero).
__device__ __forceinline__ u4_t wload(const GLOBAL uint8_t* wrow, int c, int q, int rbytes) {
  const int off = min(c * 64 + q * 16, rbytes - 16);
  return *reinterpret_cast<const GLOBAL u4_t*>(wrow + off);
}

// 0.5 * scale of this lane's four slots 4q .. 4q+3 in the window whose first
// group (relative to the range) is g0, read from this row's scales at my_sc;
// 0 where the slot is unused (activation row >= m, group past the range, row
// past n).
template <int GW>
__device__ __forceinline__ void window_scales(const uint16_t* my_sc, int g0, int ngr, int m, bool row_ok, int q,
                                              float (&s)[4]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int slot = 4 * q + v;
    const int g = g0 + slot % GW;
    const bool ok = row_ok && slot / GW < m && g < ngr;
    const uint16_t raw = my_sc[min(g, ngr - 1)];
    s[v] = ok ? 0.5f * h2f(raw) : 0.f;
  }
}

constexpr int kThreads = kWave * kWaves;

// The 16 bytes of scales at address ca (16-byte aligned); halves outside the
// scale array [s0, send) are zero and never read from memory.
__device__ __forceinline__ u4_t scale_chunk(const GLOBAL uint16_t* s0, uintptr_t send, uintptr_t ca) {
  if (ca >= (uintptr_t)s0 && ca + 16 <= send) return *reinterpret_cast<const GLOBAL u4_t*>(ca);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int i = 0; i < 8; ++i) {
    const uintptr_t a = ca + 2 * i;
    if (a >= (uintptr_t)s0 && a < send) w[i / 2] |= (uint32_t)*reinterpret_cast<const GLOBAL uint16_t*>(a) << (16 * (i % 2));
  }
  return u4_t{w[0], w[1], w[2], w[3]};
}

// Bits [lo, hi) of a 32-bit mask word (lo, hi clamped to 0..32).
__device__ __forceinline__ uint32_t range_bits(int lo, int hi) {
  lo = max(lo, 0);
  hi = min(hi, 32);
  if (hi <= lo) return 0u;
  const uint32_t upto = hi >= 32 ? ~0u : ((1u << hi) - 1u);
  return upto & ~((1u << lo) - 1u);
}

// Activation row of staging chunk id (chunks of cpr per row), without a division.
template <int MP>
__device__ __forceinline__ int xrow_of(int id, int cpr) {
  int m = 0;
#pragma unroll
  for (int j = 1; j < MP; ++j) m += id >= j * cpr ? 1 : 0;
  return m;
}

// One lane's quarter of a residual block (G/4 bytes / 4): 8 bytes for G = 128,
// 4 bytes for G = 64, and its MFMA B operands (G / 32 of them).
template <int G> struct ResQ;
template <> struct ResQ<128> { typedef u2_t T; };
template <> struct ResQ<64> { typedef uint32_t T; };

__device__ __forceinline__ void decode_quarter(u2_t v, h8_t* bb) { decode_two(v.x, v.y, bb); }
__device__ __forceinline__ void decode_quarter(uint32_t v, h8_t* bb) {
  h8_t t[4];
  decode_two(v, 0u, t);
  bb[0] = t[0];
  bb[1] = t[1];
}

// LDS staging of a work item once its small operands have arrived: scales
// (flat 16-byte chunks, or per row for a K split), activations (zero past
// the range) and the zero area.
template <int MP, int KSF>
__device__ __forceinline__ void stage_lds(uint8_t* lds, uint32_t scoff, uint32_t xoff, bool sflat, int nsch,
                                          const u4_t (&sv)[KSF], const GLOBAL uint16_t* s0, uintptr_t send,
                                          uintptr_t sa0, int ngr, int rw, int spitch, int row0, int n, int ng,
                                          int ga, int nx, int cpr, int krp, int kr, const u4_t (&xv)[8], int tid) {
  uint16_t* ssm = reinterpret_cast<uint16_t*>(lds + scoff);
  if (sflat) {
#pragma unroll
    for (int u = 0; u < KSF; ++u)
      if (u * kThreads + tid < nsch) *reinterpret_cast<u4_t*>(lds + scoff + (u * kThreads + tid) * 16) = sv[u];
    for (int c = KSF * kThreads + tid; c < nsch; c += kThreads)  // long ranges
      *reinterpret_cast<u4_t*>(lds + scoff + c * 16) = scale_chunk(s0, send, sa0 + (size_t)c * 16);
  } else {
    // K split: the item's groups of each row (thread -> groups 32c + sgl, rows srr + 8u)
    const int sgl = tid % 32, srr = tid / 32;
    for (int c = 0; c * 32 < ngr; ++c) {
      const int g = c * 32 + sgl;
      if (g < ngr)
        for (int u = 0; u < rw / 8; ++u)
          ssm[(srr + 8 * u) * spitch + g] = s0[(size_t)min(row0 + srr + 8 * u, n - 1) * ng + ga + g];
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int id = u * kThreads + tid;
    if (u * kThreads < nx && id < nx) {
      const int m = xrow_of<MP>(id, cpr);
      const int kk = (id - m * cpr) * 8;
      *reinterpret_cast<u4_t*>(lds + xoff + (size_t)m * krp * 2 + kk * 2) = kk < kr ? xv[u] : u4_t{0u, 0u, 0u, 0u};
    }
  }
  if (tid < kZeroBytes / 16) *reinterpret_cast<u4_t*>(lds + tid * 16) = u4_t{0u, 0u, 0u, 0u};
}

template <int MP>
struct Win {
  static constexpr int GW = 16 / MP;                        // groups per window
  static constexpr int NACC = GW == 2 ? 2 : 1;              // accumulators per lane
};

// LDS layout of a workgroup (byte offsets):
//   [0, 128)                       zeros
//   [128, 128 + m*KRP*2)           activations of the range, row m at m*KRP*2
//   then                           scales of the 64 rows (see stage 2)
//   then per wavefront             residual entries (kResCap x 8 B) and values
//   then                           per-group activation sums (offsets only)
static_assert(kWaves * kResCap >= kResStage, "the value area holds every staged entry");
template <int MP>
constexpr int res_wave_bytes() { return kResCap * 8 + kResCap * MP * 4; }
// staged residual entries: blocks (G/4 bytes each), then index chunks
template <int G>
constexpr int res_stage_bytes() { return kResStage * (G / 4) + (kResStage / 4 + 1) * 16; }

template <int G, int MP>
__global__ __launch_bounds__(kWave * kWaves) __attribute__((amdgpu_waves_per_eu(MP == 8 || (G == 64 && MP == 4) ? 2 : 3, 8)))
void gemv_mfma_kernel(const GemvDesc* __restrict__ descs, int ndesc, GemvDesc one) {
  constexpr int GW = Win<MP>::GW;
  constexpr int NACC = Win<MP>::NACC;
  constexpr int GPB = kBlockTrits / G;      // groups per block
  constexpr int BW = GW / GPB;              // blocks per window
  static_assert(BW >= 1, "a window must hold at least one block");
  typedef typename ResQ<G>::T RB;
  extern __shared__ uint4 smem_all[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem_all);

  // one descriptor per work item (grouped launches), or the single one
  GemvDesc d;
  if (ndesc > 0) d = descs[blockIdx.x];
  else d = one;
  const int item = (int)blockIdx.x - d.tile_begin;
  const int rb = item % d.row_blocks;
  const int split = item / d.row_blocks;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int q = lane / 16, r = lane % 16;
  // kw wavefronts share a 16-row tile, each taking a part of the K range
  const int kw = d.kwaves;
  const int rw = kRowsWave * (kWaves / kw);   // rows per work item
  const int tile = wave / kw, kp = wave % kw;
  const int row0 = rb * rw;
  const int row = row0 + tile * kRowsWave + r;
  const bool row_ok = row < d.n;
  const int rowc = row_ok ? row : d.n - 1;  // clamped: loads stay in bounds
  const int dm = d.m;
  // the item's groups [ga, gb); this wavefront's part [pga, pgb) in whole blocks
  const int ga = split * d.gps;
  const int gb = min(d.ng, ga + d.gps);
  const int k0 = ga * G;
  const int kr = (gb - ga) * G;                       // trits of the item (multiple of 64)
  const int nblk_i = (kr + kBlockTrits - 1) / kBlockTrits;
  const int krp = nblk_i * kBlockTrits;               // padded range in LDS
  const int ngr = gb - ga;
  const int bpp = (nblk_i + kw - 1) / kw;
  const int pb0 = min(nblk_i, kp * bpp), pb1 = min(nblk_i, pb0 + bpp);
  const int nblk = pb1 - pb0;                          // this wavefront's blocks (may be 0)
  const int pga = ga + pb0 * GPB, pgb = min(gb, ga + pb1 * GPB);
  // scales in LDS: rows of `spitch` groups; whole rows copied as raw 16-byte
  // chunks when K is not split (flat), else the item's groups of each row
  const bool sflat = ga == 0 && gb == d.ng;
  const int spitch = sflat ? d.ng : ngr;
  const uint32_t xoff = kZeroBytes;                                            // activations
  const uint32_t scoff = xoff + (uint32_t)dm * krp * 2;                        // scales
  const uint32_t scbytes = ((uint32_t)kGemvRows * spitch * 2 + 32 + 15) / 16 * 16;  // + chunk slack
  // residual values [4 waves][kResCap][MP] (a tile's kw waves are adjacent,
  // so a tile owns kw * kResCap consecutive entries), then entry lists
  const uint32_t valoff = scoff + scbytes;
  const uint32_t entoff = valoff + kWaves * kResCap * MP * 4 + (uint32_t)wave * kResCap * 8;
  const uint32_t rstoff = valoff + kWaves * res_wave_bytes<MP>();              // staged residual data
  const uint32_t redoff = rstoff + res_stage_bytes<G>();                       // part sums
  const uint32_t soff = redoff + kWaves * MP * kRowsWave * 4;                  // group sums of x

  // bytes of this wavefront's part in one row (an empty part reads, and
  // ignores, the item's first 16 bytes, so the loads are unconditional)
  const int rbytes = max((pgb - pga) * G / 4, 16);
  const GLOBAL uint8_t* wrow = gp(d.plane0) + (size_t)rowc * d.stride + (k0 + pb0 * kBlockTrits) / 4;
  const GLOBAL uint16_t* s0 = gp(d.scale0);
  const int cpr = krp / 8;   // 16-byte activation chunks per activation row
  const int nx = dm * cpr;   // at most 2048: MP * krp <= 16384

  // ---- 1. loads of the small operands, then the first weights; only the
  // small operands are waited for before the main loop
  // scales, flat: 16-byte chunks covering this item's rows (they are
  // contiguous), from the 16-byte boundary at or below the first scale
  const uintptr_t sfirst = (uintptr_t)(s0 + (size_t)row0 * d.ng);
  const uintptr_t sa0 = sfirst & ~(uintptr_t)15;
  const int sshift = (int)(sfirst - sa0) / 2;  // elements before row0's first scale
  const int nsch = sflat ? (int)(((uintptr_t)(s0 + (size_t)min(row0 + rw, d.n) * d.ng) - sa0 + 15) / 16) : 0;
  constexpr int kSF = 4;  // chunk rounds loaded ahead (more are staged afterwards)
  const uintptr_t send = (uintptr_t)(s0 + (size_t)d.n * d.ng);  // end of the scale array
  u4_t sv[kSF];
#pragma unroll
  for (int u = 0; u < kSF; ++u)
    if (u * kThreads < nsch) sv[u] = scale_chunk(s0, send, sa0 + (size_t)min(u * kThreads + tid, nsch - 1) * 16);
  // activations [dm][krp] (one round always suffices)
  u4_t xv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (u * kThreads < nx) {
      const int id = min(u * kThreads + tid, nx - 1);
      const int m = xrow_of<MP>(id, cpr);
      const int kk = min((id - m * cpr) * 8, kr - 8);
      xv[u] = *reinterpret_cast<const GLOBAL u4_t*>(gp(d.x) + (size_t)m * d.k + k0 + kk);
    }
  }
  // first residual plane, when the plan indexed it and the item covers the
  // whole row: the workgroup's entries [e0, e1) (its rows are contiguous) are
  // staged in LDS with the other small operands -- their blocks as raw
  // 16-byte chunks and their index words (group | scale bits << 16)
  uint32_t e0 = 0, e1 = 0;
  if (d.gidx[0] != nullptr && sflat && d.planes == 2) {
    const int nt = rw / kRowsWave;
    e0 = d.tile_e[0][0];
    e1 = nt == 1 ? d.tile_e[0][1] : nt == 2 ? d.tile_e[0][2] : d.tile_e[0][4];
  }
  const bool res_idx = e1 > e0 && e1 - e0 <= (uint32_t)kResStage;
  const uint32_t nres = res_idx ? e1 - e0 : 0u;
  constexpr int kBQ = G / 4 / 16;                          // 16-byte chunks per block
  const GLOBAL uint32_t* gix = gp(d.gidx[0]);
  const uintptr_t gfirst = (uintptr_t)(gix + e0), ga0 = gfirst & ~(uintptr_t)15;
  const int gshift = (int)(gfirst - ga0) / 4;
  const int nbch = (int)nres * kBQ;                        // block chunks
  const int ngch = res_idx ? (int)(((uintptr_t)(gix + e1) - ga0 + 15) / 16) : 0;  // index chunks
  constexpr int kRS = (kResStage * kBQ + kResStage / 4 + 1 + kThreads - 1) / kThreads;
  u4_t rv[kRS];
#pragma unroll
  for (int u = 0; u < kRS; ++u) {
    if (u * kThreads < nbch + ngch) {
      const int c = min(u * kThreads + tid, nbch + ngch - 1);
      if (c < nbch)
        rv[u] = *reinterpret_cast<const GLOBAL u4_t*>(gp(d.blocks[0]) + ((size_t)e0 * kBQ + c) * 16);
      else
        rv[u] = *reinterpret_cast<const GLOBAL u4_t*>(ga0 + (size_t)(c - nbch) * 16);
    }
  }
  // this row's entries, for the sums
  uint32_t rp0 = 0, rp1 = 0;
  if (res_idx) {
    rp0 = gp(d.rowptr[0])[rowc];
    rp1 = gp(d.rowptr[0])[rowc + 1];
  }

  float* valw = reinterpret_cast<float*>(lds + valoff) + (size_t)wave * kResCap * MP;  // this wave's
  float* valr = reinterpret_cast<float*>(lds + valoff);  // staged entries' values [entry][m]
  uint32_t* ent = reinterpret_cast<uint32_t*>(lds + entoff);

  // this lane's slot: activation row m_a = r / GW, group offset r % GW in the window
  const int m_a = r / GW;
  const bool a_row = m_a < dm;
  const uint32_t abase = xoff + (uint32_t)(m_a * krp + pb0 * kBlockTrits + q * 64) * 2;
  float acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = 0.f;
  f4_t D = {0.f, 0.f, 0.f, 0.f}, E = {0.f, 0.f, 0.f, 0.f};  // even / odd MFMAs of a block
  // this row's scales from the part's first group on
  const uint16_t* my_sc = reinterpret_cast<const uint16_t*>(lds + scoff) + (sflat ? sshift : 0) +
                          (tile * kRowsWave + r) * spitch + (pga - (sflat ? 0 : ga));
  const int ngp = pgb - pga;
  // an empty part reads, and ignores, the item's first 16 bytes
  const GLOBAL uint8_t* wr = nblk > 0 ? wrow : wrow - (pb0 * kBlockTrits) / 4;

  // One 16-entry batch: entry t = b0 + r (t < wn) has block quarter BLKQ and
  // group GRR (relative to the item's range); its scaled partial sums go to
  // val[t][m].
#define TERN_RES_BATCH(VAL, B0, WN, BLKQ, GRR, RSV)                                           \
  do {                                                                                        \
    const uint32_t t_ = (B0) + r;                                                             \
    const bool ok_ = t_ < (WN);                                                               \
    h8_t bb_[4];                                                                              \
    decode_quarter(ok_ ? (BLKQ) : RB{}, bb_);                                                 \
    _Pragma("unroll") for (int m = 0; m < MP; ++m) {                                          \
      if (m < dm) {                                                                           \
        f4_t R_ = {0.f, 0.f, 0.f, 0.f};                                                       \
        const uint32_t ab_ = ok_ ? xoff + (uint32_t)(m * krp + (GRR) * G + q * (G / 4)) * 2 : 0u; \
        _Pragma("unroll") for (int j = 0; j < G / 32; ++j)                                    \
          R_ = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_h8(lds, ab_ + 16u * j), bb_[j], R_, 0, 0, 0); \
        /* diagonal: entry r sits in lane 16 * (r / 4) + r, element r % 4 */                  \
        if (q == r / 4 && ok_) (VAL)[t_ * MP + m] = (RSV) * R_[r % 4];                        \
      }                                                                                       \
    }                                                                                         \
  } while (0)
  // each owner adds its row's entries of the window [W0, W0 + WN) in order
#define TERN_RES_SUM(PRE, CNT, W0, WN)                                                        \
  do {                                                                                        \
    const uint32_t lo_ = max((PRE), (W0)), hi_ = min((PRE) + (CNT), (W0) + (WN));             \
    _Pragma("unroll") for (int i = 0; i < NACC; ++i)                                          \
      if (owner && m_of[i] < dm)                                                              \
        for (uint32_t e = lo_; e < hi_; ++e) acc[i] += valw[(e - (W0)) * MP + m_of[i]];       \
  } while (0)

  // One block: decode, 8 MFMAs.  Window boundaries are static in the
  // unrolled body because BW divides 8.
#define TERN_BLOCK(V, C, I)                                                                   \
  do {                                                                                        \
    const int wc_ = (I) % BW;                                                                 \
    const int grel_ = GPB * wc_ + q / (4 / GPB);                                              \
    const bool act_ = a_row && (r % GW) == grel_;                                             \
    const uint32_t aoff_ = act_ ? abase + (uint32_t)(C) * (kBlockTrits * 2) : 0u;             \
    h8_t b_[8];                                                                               \
    decode_two((V).x, (V).y, &b_[0]);                                                         \
    decode_two((V).z, (V).w, &b_[4]);                                                         \
    _Pragma("unroll") for (int j = 0; j < 8; j += 2) {                                        \
      D = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_h8(lds, aoff_ + 16u * j), b_[j], D, 0, 0, 0); \
      E = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_h8(lds, aoff_ + 16u * (j + 1)), b_[j + 1], E, 0, 0, 0); \
    }                                                                                         \
    __builtin_amdgcn_sched_barrier(0); /* one block's operands live at a time */              \
  } while (0)
  // close window wi: scale the slot sums, start the next window
#define TERN_CLOSE(WI)                                                                        \
  do {                                                                                        \
    float sc_[4];                                                                             \
    window_scales<GW>(my_sc, (WI) * GW, ngp, dm, row_ok, q, sc_);                             \
    _Pragma("unroll") for (int v = 0; v < 4; ++v)                                             \
      acc[NACC == 2 ? v / 2 : 0] = fmaf(sc_[v], D[v] + E[v], acc[NACC == 2 ? v / 2 : 0]);     \
    D = f4_t{0.f, 0.f, 0.f, 0.f};                                                             \
    E = f4_t{0.f, 0.f, 0.f, 0.f};                                                             \
  } while (0)

  // ---- 2..5 with NB weight loads in flight.  Every wavefront's blocks (at
  // most bpp <= kMaxBlocks: the host chooses kwaves and splits so) are requested at once, right
  // after the small operands; loads past a wavefront's blocks repeat its last
  // block.  NB is uniform over the workgroup (bpp), so every wavefront meets
  // the same barrier.
#define TERN_BODY(NB)                                                                         \
  do {                                                                                        \
    u4_t w_[NB];                                                                              \
    stage_lds<MP, kSF>(lds, scoff, xoff, sflat, nsch, sv, s0, send, sa0, ngr, rw, spitch, row0,         \
              d.n, d.ng, ga, nx, cpr, krp, kr, xv, tid);                                      \
    _Pragma("unroll") for (int u = 0; u < kRS; ++u) {                                         \
      const int c_ = u * kThreads + tid;                                                      \
      if (u * kThreads < nbch + ngch && c_ < nbch + ngch)                                     \
        *reinterpret_cast<u4_t*>(lds + rstoff + (c_ < nbch ? c_ * 16 : kResStage * (G / 4) + (c_ - nbch) * 16)) = rv[u]; \
    }                                                                                         \
    __syncthreads();                                                                          \
    /* the weights, once the small operands have landed (issued earlier they */               \
    /* would queue the small operands behind every wavefront's weights) */                    \
    _Pragma("unroll") for (int i = 0; i < NB; ++i) w_[i] = wload(wr, min(i, max(nblk - 1, 0)), q, rbytes); \
    /* residual batches of the staged entries, spread over the wavefronts */                 \
    for (uint32_t b0_ = 16u * wave; b0_ < nres; b0_ += 16u * kWaves) {                         \
      const uint32_t t_ = min(b0_ + r, nres - 1);                                             \
      const RB bq_ = *reinterpret_cast<const RB*>(lds + rstoff + t_ * (G / 4) + q * sizeof(RB)); \
      const uint32_t gi_ = *reinterpret_cast<const uint32_t*>(lds + rstoff + kResStage * (G / 4) + (gshift + t_) * 4); \
      TERN_RES_BATCH(valr, b0_, nres, bq_, (int)(gi_ & 0xFFFFu), 0.5f * h2f((uint16_t)(gi_ >> 16))); \
    }                                                                                         \
    /* plane 0 */                                                                             \
    _Pragma("unroll") for (int i = 0; i < NB; ++i) {                                          \
      if (i < nblk) {                                                                         \
        TERN_BLOCK(w_[i], i, i);                                                              \
        if (i % BW == BW - 1) TERN_CLOSE(i / BW);                                             \
      }                                                                                       \
    }                                                                                         \
    if (nblk > 0 && nblk % BW != 0) TERN_CLOSE((nblk - 1) / BW);                              \
  } while (0)
  if (bpp > 8) TERN_BODY(kMaxBlocks);
  else TERN_BODY(8);
#undef TERN_BODY
#undef TERN_BLOCK
#undef TERN_CLOSE

  // sum the lanes that hold other groups of the same (row, activation row)
  if (GW >= 8) acc[0] += __shfl_xor(acc[0], 16, kWave);
  if (GW >= 16) acc[0] += __shfl_xor(acc[0], 32, kWave);
  // owner lanes: activation row of acc[i]
  int m_of[NACC];
  bool owner;
  if (GW == 16) { m_of[0] = 0; owner = q == 0; }
  else if (GW == 8) { m_of[0] = q / 2; owner = (q % 2) == 0; }
  else if (GW == 4) { m_of[0] = q; owner = true; }
  else { m_of[0] = 2 * q; m_of[NACC - 1] = 2 * q + 1; owner = true; }

  // ---- residual planes over [pga, pgb)
  for (int p = 0; p + 1 < d.planes && pgb > pga; ++p) {
    const GLOBAL uint8_t* blocks = gp(p == 0 ? d.blocks[0] : d.blocks[1]);
    const GLOBAL uint16_t* rscale = gp(p == 0 ? d.rscale[0] : d.rscale[1]);
    const uint32_t w_begin = 0;
    if (p == 0 && res_idx) continue;  // done before plane 0
    // general path: list from the mask in global memory, window by window
    const int wlo = pga >> 5, whi = (pgb - 1) >> 5;
    const GLOBAL uint32_t* mrow = gp(p == 0 ? d.mask[0] : d.mask[1]) + (size_t)rowc * d.mwords;
    uint32_t base = 0, cnt = 0;
    if (row_ok) {
      base = gp(p == 0 ? d.rowptr[0] : d.rowptr[1])[row];
      for (int w = 0; w < wlo; ++w) base += __popc(mrow[w]);
      if (pga & 31) base += __popc(mrow[wlo] & ((1u << (pga & 31)) - 1u));
      for (int w = wlo; w <= whi; ++w) cnt += __popc(mrow[w] & range_bits(pga - (w << 5), pgb - (w << 5)));
    }
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o, 16);
      if (r >= o) incl += t;
    }
    const uint32_t pre_r = incl - cnt;
    const uint32_t total = __shfl(incl, 15, kWave);
    for (uint32_t w0 = w_begin; w0 < total; w0 += kResCap) {
      const uint32_t wn = min((uint32_t)kResCap, total - w0);
      wave_sync();
      if (q == 0 && cnt && pre_r < w0 + wn && pre_r + cnt > w0) {
        uint32_t e = pre_r;
        for (int w = wlo; w <= whi; ++w) {
          uint32_t bits = mrow[w] & range_bits(pga - (w << 5), pgb - (w << 5));
          while (bits) {
            const int g = (w << 5) + __builtin_ctz(bits);
            bits &= bits - 1u;
            if (e >= w0 && e < w0 + wn) {
              ent[2 * (e - w0)] = base + (e - pre_r);
              ent[2 * (e - w0) + 1] = (uint32_t)(g - ga);
            }
            ++e;
          }
        }
      }
      wave_sync();
      for (uint32_t b0 = 0; b0 < wn; b0 += 16) {
        const uint32_t t = b0 + r;
        const uint32_t blk = t < wn ? ent[2 * t] : 0u;
        const int grr = t < wn ? (int)ent[2 * t + 1] : 0;
        const RB bq = *reinterpret_cast<const GLOBAL RB*>(blocks + (size_t)blk * (G / 4) + q * sizeof(RB));
        const float rs = t < wn ? 0.5f * h2f(rscale[blk]) : 0.f;
        TERN_RES_BATCH(valw, b0, wn, bq, grr, rs);
      }
      wave_sync();
      if (cnt) TERN_RES_SUM(pre_r, cnt, w0, wn);
    }
  }
#undef TERN_RES_BATCH
#undef TERN_RES_SUM

  // ---- per-group activation sums for the offsets (once per workgroup)
  float* xsum = reinterpret_cast<float*>(lds + soff);
  if (d.offset_mode != 0) {
    for (int id = tid; id < dm * ngr; id += kThreads) {
      const int m = id / ngr, g = id % ngr;
      const uint32_t* xw = reinterpret_cast<const uint32_t*>(lds + xoff + (size_t)(m * krp + g * G) * 2);
      float s = 0.f;
      for (int i = 0; i < G / 2; ++i)
        s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, xw[i]), h2_t{(_Float16)1.f, (_Float16)1.f}, s, false);
      xsum[id] = s;
    }
  }
  // ---- the parts of a row tile, summed in part order
  float* red = reinterpret_cast<float*>(lds + redoff);
  if (kw > 1) {
#pragma unroll
    for (int i = 0; i < NACC; ++i)
      if (owner && m_of[i] < dm) red[(wave * MP + m_of[i]) * kRowsWave + r] = acc[i];
  }
  if (kw > 1 || d.offset_mode != 0 || res_idx) __syncthreads();
  if (kp != 0) return;
  if (kw > 1) {
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
      if (owner && m_of[i] < dm) {
        float v = red[((tile * kw) * MP + m_of[i]) * kRowsWave + r];
        for (int pp = 1; pp < kw; ++pp) v += red[((tile * kw + pp) * MP + m_of[i]) * kRowsWave + r];
        acc[i] = v;
      }
    }
  }
  // staged residual entries of this row: the row's four lanes take every
  // fourth entry, then the quarters are added (fixed order)
  if (res_idx) {
    float rsum[MP];
#pragma unroll
    for (int m = 0; m < MP; ++m) rsum[m] = 0.f;
    if (row_ok)
      for (uint32_t e = rp0 + q; e < rp1; e += 4)
#pragma unroll
        for (int m = 0; m < MP; ++m) rsum[m] += valr[(e - e0) * MP + m];
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      rsum[m] += __shfl_xor(rsum[m], 16, kWave);
      rsum[m] += __shfl_xor(rsum[m], 32, kWave);
    }
#pragma unroll
    for (int i = 0; i < NACC; ++i)
      if (owner && m_of[i] < dm) {
        float v = 0.f;
#pragma unroll
        for (int m = 0; m < MP; ++m) v = m == m_of[i] ? rsum[m] : v;
        acc[i] += v;
      }
  }
  // ---- offsets over the item's range
  if (d.offset_mode != 0) {
    const GLOBAL uint16_t* off = gp(d.offset);
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
      if (owner && row_ok && m_of[i] < dm) {
        const float* xs = xsum + m_of[i] * ngr;
        if (d.offset_mode == 1) {
          float s = 0.f;
          for (int g = 0; g < ngr; ++g) s += xs[g];
          acc[i] = fmaf(h2f(off[row]), s, acc[i]);
        } else {
          const GLOBAL uint16_t* orow = off + (size_t)row * d.ng + ga;
          for (int g = 0; g < ngr; ++g) acc[i] = fmaf(h2f(orow[g]), xs[g], acc[i]);
        }
      }
    }
  }

  // ---- output
  if (!owner || !row_ok) return;
#pragma unroll
  for (int i = 0; i < NACC; ++i) {
    const int m = m_of[i];
    if (m < dm) {
      if (d.splits > 1)
        d.partial[((size_t)split * dm + m) * d.n + row] = acc[i];
      else if (d.y_f32)
        reinterpret_cast<float*>(d.y)[(size_t)m * d.n + row] = acc[i];
      else
        reinterpret_cast<_Float16*>(d.y)[(size_t)m * d.n + row] = (_Float16)acc[i];
    }
  }
}

template <int G, int MP>
hipError_t launch_mfma(const GemvDesc* descs, int ndesc, const GemvDesc& one, int items, int max_krp, bool offsets,
                       hipStream_t s) {
  const int ngr = max_krp / G;
  size_t lds = kZeroBytes + (size_t)MP * max_krp * 2 + ((size_t)kGemvRows * ngr * 2 + 32 + 15) / 16 * 16 +
               (size_t)kWaves * res_wave_bytes<MP>() + res_stage_bytes<G>() + (size_t)kWaves * MP * kRowsWave * 4;
  if (offsets) lds += (size_t)MP * (max_krp / G) * 4;
  hipLaunchKernelGGL((gemv_mfma_kernel<G, MP>), dim3(items), dim3(kWave * kWaves), lds, s, descs, ndesc, one);
  return hipGetLastError();
}

template <int G>
hipError_t launch_mfma_g(int mp, const GemvDesc* descs, int ndesc, const GemvDesc& one, int items, int max_krp,
                         bool offsets, hipStream_t s) {
  switch (mp) {
    case 1: return launch_mfma<G, 1>(descs, ndesc, one, items, max_krp, offsets, s);
    case 2: return launch_mfma<G, 2>(descs, ndesc, one, items, max_krp, offsets, s);
    case 4: return launch_mfma<G, 4>(descs, ndesc, one, items, max_krp, offsets, s);
    case 8:
      if (G == 128) return launch_mfma<128, 8>(descs, ndesc, one, items, max_krp, offsets, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

__global__ void res_index_kernel(const uint32_t* __restrict__ mask, const uint32_t* __restrict__ rowptr,
                                 const uint16_t* __restrict__ rscale, int n, int mwords,
                                 uint32_t* __restrict__ gidx) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n) return;
  uint32_t e = rowptr[row];
  for (int w = 0; w < mwords; ++w) {
    uint32_t bits = mask[(size_t)row * mwords + w];
    while (bits) {
      gidx[e] = (uint32_t)(32 * w + __builtin_ctz(bits)) | ((uint32_t)rscale[e] << 16);
      ++e;
      bits &= bits - 1u;
    }
  }
}

__global__ void tile_bounds_kernel(GemvDesc* items, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  GemvDesc* d = items + i;
  const int item = i - d->tile_begin;
  const int row0 = (item % d->row_blocks) * kRowsWave * (kWaves / d->kwaves);
  for (int p = 0; p < 2; ++p) {
    if (!d->gidx[p]) continue;
    for (int t = 0; t < 5; ++t) d->tile_e[p][t] = d->rowptr[p][min(row0 + kRowsWave * t, d->n)];
  }
}

}  // namespace

hipError_t launch_res_index(const uint32_t* mask, const uint32_t* rowptr, const uint16_t* rscale, int n,
                            int mwords, uint32_t* gidx, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(res_index_kernel, dim3((n + 255) / 256), dim3(256), 0, s, mask, rowptr, rscale, n, mwords,
                     gidx);
  return hipGetLastError();
}

hipError_t launch_tile_bounds(GemvDesc* items, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(tile_bounds_kernel, dim3((count + 255) / 256), dim3(256), 0, s, items, count);
  return hipGetLastError();
}

int gemv_mfma_max_rows(int group) { return group == 128 ? 8 : 4; }

int gemv_mfma_max_range(int mp) { return std::min(16384 / mp, kMaxBlocks * kBlockTrits * kWaves); }

hipError_t launch_gemv_mfma(int group, int mp, const GemvDesc* descs, int ndesc, const GemvDesc& one,
                            int total_items, int max_krp, bool offsets, hipStream_t s) {
  if (total_items <= 0) return hipSuccess;
  if (group == 64) return launch_mfma_g<64>(mp, descs, ndesc, one, total_items, max_krp, offsets, s);
  if (group == 128) return launch_mfma_g<128>(mp, descs, ndesc, one, total_items, max_krp, offsets, s);
  return hipErrorInvalidValue;
}

}  // namespace tern
