// Batched product y = x W^T for many activation rows (tuned for M >= 64):
// packed weights are decoded into an FP16 tile in LDS
// (W~[n,k] = off + s0*t0 + m1*s1*t1 + m2*s2*t2, stored doubled), and the tile
// product runs on the matrix cores (v_mfma_f32_32x32x16_f16, FP32
// accumulation).  This is the batched-execution direction named by arXiv
// 2609.09240 (kernel optimisation across shapes and batch sizes); at M >= 64
// the product is a dense contraction, so MFMA is the right unit.
//
// Tile: BM activation rows (256, or 128 for small M) x 128 weight rows, K in
// steps of 64.  256 threads = 4 waves in a 2 x 2 arrangement; a wave owns
// BM/2 x 64 outputs as (BM/64) x 2 MFMA tiles of 32 x 32.  Each step stages
// the activation tile (copied) and the weight tile (decoded: thread = one
// weight row and 32 of the step's 64 trits) in one of two LDS buffers, so one
// barrier per step separates staging from the products, and the next step's
// global loads are in flight while this step's products run.
// Operand layout of the 32x32x16 f16 MFMA: lane l supplies A[l%32][8*(l/32)
// .. +7] and B[8*(l/32) .. +7][l%32] and receives D[8*(v/4) + 4*(l/32) +
// v%4][l%32], v = 0..15.
#include <algorithm>

#include "internal.h"

namespace tern {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));

constexpr int NT = 256;     // threads per workgroup
constexpr int BN = 128;     // weight rows per tile
constexpr int BK = 64;      // K per step
constexpr int PH = BK + 8;  // LDS row pitch in halves: 144 B keeps 16-lane 16-byte accesses conflict-free

// FP16 pair (2*t[2i], 2*t[2i+1]) of 2-bit word w (see the decode kernel).
__device__ __forceinline__ uint32_t pair_of(uint32_t w, int shift) { return (w << shift) & 0xC000C000u; }

__device__ __forceinline__ uint32_t pk_mul(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, a) * __builtin_bit_cast(h2_t, b));
}
__device__ __forceinline__ uint32_t pk_fma(uint32_t a, uint32_t b, uint32_t c) {
  const h2_t r = __builtin_bit_cast(h2_t, a) * __builtin_bit_cast(h2_t, b) + __builtin_bit_cast(h2_t, c);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pk_add(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, a) + __builtin_bit_cast(h2_t, b));
}
__device__ __forceinline__ uint32_t splat(uint32_t h) { return (h & 0xFFFFu) * 0x10001u; }
__device__ __forceinline__ float h2f_bits(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// Base-3 byte -> five 2-bit codes at bits 0..9 (trit i at bits 2i..2i+1).
__device__ __forceinline__ uint32_t b3_codes(uint32_t v) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    c |= ((uint32_t)((int)(v % 3u) - 1) & 3u) << (2 * i);
    v /= 3u;
  }
  return c;
}

// Buffer resource over `bytes` bytes at p: loads at or past the end return 0,
// which zeroes the operands of rows past n or m without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Buffer resources and per-thread offsets of one matrix.
struct Src {
  __amdgpu_buffer_rsrc_t p0, sc, offg, mask[2], blk[2], rsc[2];
  uint32_t sc_v, offg_v, mask_v;  // row-dependent byte offsets of the decoding thread's row
};

// Packed plane-0 bytes reach LDS in windows of WSTEPS steps: every row of the
// tile loads WB bytes with coalesced 16-byte loads (2-bit: 4 steps = 64 B;
// base-3: 4 steps = 52 B from a dword boundary, read as 64).  Three window
// buffers let each pair of steps load and store one chunk per thread.
constexpr int WSTEPS = 4;
constexpr int WB = 64;
constexpr int WP = WB + 16;             // LDS pitch of a window row
constexpr int NWIN = 3;
constexpr int WCH = BN * WB / 16 / NT;  // 16-byte window chunks per thread and window (2)
constexpr uint32_t kOOB = 0x7FFFFFF0u;  // offset past every buffer: the load returns zero

template <int FMT>
__device__ __forceinline__ int win_start(int w) { return FMT == 0 ? WB * w : 52 * w; }

// Per-step operands of one thread (scale, per-group offset, residual), loaded
// a step ahead of their decode.  Residual loads of lanes whose row has no
// block at the group use an out-of-range offset, so every step issues the
// same loads.
template <int NP>
struct Pre {
  uint32_t s0;                       // plane-0 scale (FP16 bits; 0 past row n)
  uint32_t off;                      // per-group offset (FP16 bits; 0 unless per-group offsets)
  uint32_t has;                      // bit p: residual plane p+1 present at the group
  uint32_t rw[NP > 0 ? NP : 1][2];   // residual 2-bit words of the thread's 32 trits
  uint32_t rs[NP > 0 ? NP : 1];      // residual scales
};

// Residual walk of the decoding thread's row, kept at the group of the last
// issued step loads: e[p] = entry index of that group's block (if present),
// mwl[p] = the mask word holding that group, mwn[p] = the next mask word
// (reloaded every other step).
template <int NP>
struct Walk {
  uint32_t e[NP > 0 ? NP : 1], mwl[NP > 0 ? NP : 1], mwn[NP > 0 ? NP : 1];
};

// gc = g clamped to the last group (steps past the end reload it).
template <int G, int NP, int A>
__device__ __forceinline__ void load_step(const Src& S, int g, int gc, const Walk<NP>& W, Pre<NP>& P) {
  P.s0 = __builtin_amdgcn_raw_buffer_load_b16(S.sc, S.sc_v, 2 * gc, 0);
  P.off = __builtin_amdgcn_raw_buffer_load_b16(S.offg, S.offg_v, 2 * gc, 0);
  P.has = 0;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const uint32_t pr = (W.mwl[p] >> (g & 31)) & 1u;
    P.has |= pr << p;
    P.rs[p] = __builtin_amdgcn_raw_buffer_load_b16(S.rsc[p], pr ? 2 * W.e[p] : kOOB, 0, 0);
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(S.blk[p], pr ? W.e[p] * (G / 4) + A / 4 : kOOB, 0, 0);
    P.rw[p][0] = v[0];
    P.rw[p][1] = v[1];
  }
}

// Moves the walk from group g to group g + 1.
template <int NP>
__device__ __forceinline__ void walk_next(int g, Walk<NP>& W) {
#pragma unroll
  for (int p = 0; p < NP; ++p) W.e[p] += (W.mwl[p] >> (g & 31)) & 1u;
  if (((g + 1) & 31) == 0) {
#pragma unroll
    for (int p = 0; p < NP; ++p) W.mwl[p] = W.mwn[p];
  }
}

// The decoded weights of the thread's 32 trits as 16 FP16 pairs in K order.
// Narrow (WIDE false): 2*W~ = 2*(s0*t0 + m1*s1*t1 + m2*s2*t2 + off) with FP16
// fused multiply-adds, for products whose chain rounds at most once (no
// offset and at most one residual plane, or an offset and no residual plane:
// the first multiply-add of (2t) * s is exact).  Wide: W~ formed in FP32 from
// exact products (2t) * (s/2) and rounded once to FP16, for products with an
// offset and residual planes, or two residual planes, whose FP16 chain
// would round two or three times; the tile then holds W~ instead of 2*W~ (the
// epilogue scales by 1 instead of 0.5).  prep() reads the packed bytes from
// the LDS window and takes the scales, pair(i) forms pair i, store() writes
// four pairs to LDS; the product loop calls them one piece at a time between
// its MFMAs.
template <int FMT, int G, int NP, int A, bool WIDE>
struct Dec {
  static constexpr int B0 = A / 5, NB = (A + 31) / 5 - B0 + 1;
  uint32_t out[16];
  uint32_t s0, o2, s1[NP > 0 ? NP : 1];  // narrow: FP16 pairs
  float s0h, of, s1h[NP > 0 ? NP : 1];   // wide: s0 / 2, off, s_p / 2 in FP32
  uint32_t w[FMT == 0 ? 2 : NB];  // 2-bit words, or base-3 code words
  uint32_t rw[NP > 0 ? NP : 1][2];

  // win: this thread's row in the LDS window holding step s; u = s % WSTEPS;
  // g = group of step s; wstart = first row byte of the window; ro = row
  // offset (FP16 bits; 0 unless per-row offsets)
  __device__ __forceinline__ void prep(int g, int u, int wstart, const uint8_t* win, const Pre<NP>& P,
                                       uint32_t ro, const uint32_t* lut) {
    if constexpr (WIDE) {
      s0h = 0.5f * h2f_bits(P.s0);
      of = h2f_bits(ro | P.off);  // at most one of them is non-zero
    } else {
      s0 = splat(P.s0);
      const uint32_t o = splat(ro | P.off);  // at most one of them is non-zero
      o2 = pk_add(o, o);
    }
    if constexpr (FMT == 0) {
      const uint2 v = *reinterpret_cast<const uint2*>(win + 16 * u + 8 * ((A / 32) & 1));
      w[0] = v.x;
      w[1] = v.y;
    } else {
      // bytes of trits [A, A + 32) of group g: at most 8 from byte b of the window
      constexpr int GB = (G + 4) / 5;
      const int b = g * GB + A / 5 - wstart;
      const uint32_t* wp = reinterpret_cast<const uint32_t*>(win + (b & ~3));
      const uint32_t w0 = wp[0], w1 = wp[1], w2 = wp[2];
      const uint32_t bsh = (uint32_t)(b & 3);
      const uint32_t lo = __builtin_amdgcn_alignbyte(w1, w0, bsh), hi = __builtin_amdgcn_alignbyte(w2, w1, bsh);
#pragma unroll
      for (int j = 0; j < NB; ++j) w[j] = lut[((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xFFu];
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if constexpr (WIDE) s1h[p] = ((P.has >> p) & 1u) ? 0.5f * h2f_bits(P.rs[p]) : 0.f;
      else s1[p] = ((P.has >> p) & 1u) ? splat(P.rs[p]) : 0u;
      rw[p][0] = P.rw[p][0];
      rw[p][1] = P.rw[p][1];
    }
  }

  __device__ __forceinline__ void pair(int i) {
    uint32_t t2;  // FP16 pair (2 t, 2 t') of plane 0
    if constexpr (FMT == 0) {
      t2 = pair_of(w[i >> 3], 14 - 2 * (i & 7));
    } else {
      const int ta = A + 2 * i, tb = ta + 1;
      const uint32_t ca = (w[ta / 5 - B0] >> (2 * (ta % 5))) & 3u;
      const uint32_t cb = (w[tb / 5 - B0] >> (2 * (tb % 5))) & 3u;
      t2 = (ca << 14) | (cb << 30);
    }
    if constexpr (WIDE) {
      h2_t h = __builtin_bit_cast(h2_t, t2);
      float a = fmaf((float)h.x, s0h, of), b = fmaf((float)h.y, s0h, of);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        h = __builtin_bit_cast(h2_t, pair_of(rw[p][i >> 3], 14 - 2 * (i & 7)));
        a = fmaf((float)h.x, s1h[p], a);
        b = fmaf((float)h.y, s1h[p], b);
      }
      const h2_t r = {(_Float16)a, (_Float16)b};
      out[i] = __builtin_bit_cast(uint32_t, r);
    } else {
      uint32_t v = pk_fma(t2, s0, o2);
#pragma unroll
      for (int p = 0; p < NP; ++p) v = pk_fma(pair_of(rw[p][i >> 3], 14 - 2 * (i & 7)), s1[p], v);
      out[i] = v;
    }
  }

  __device__ __forceinline__ void store(int q, _Float16* dst_h) const {
    reinterpret_cast<uint4*>(dst_h)[q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
  }
};

// dst = esc * acc for one tile of a [d.m][d.n] array of T, staged through LDS
// (the activation buffers) so that rows leave in 16-byte chunks; FP32 tiles
// of 256 rows go in two halves.
template <typename T, int AW>
__device__ __forceinline__ void epilogue(const GemvDesc& d, int m0, int n0, const f16v_t (&acc)[AW][2], char* tile,
                                         void* dst, float esc) {
  constexpr int BM = 64 * AW;
  constexpr int HALVES = (sizeof(T) == 4 && AW == 4) ? 2 : 1;
  constexpr int ROWS = BM / HALVES;
  constexpr int TP = BN * (int)sizeof(T) + 16;  // tile pitch in bytes
  constexpr int CPR = BN * (int)sizeof(T) / 16;  // 16-byte chunks per row
  constexpr int PER = 16 / (int)sizeof(T);
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int mb = (wave >> 1) * 32 * AW, nb = (wave & 1) * 64;
  const bool vec = (d.n % PER == 0) && (n0 + BN <= d.n);
#pragma unroll
  for (int hf = 0; hf < HALVES; ++hf) {
    if (HALVES == 1 || (wave >> 1) == hf) {
      char* base = tile + (mb - hf * ROWS + 4 * (lane >> 5)) * TP + (nb + (lane & 31)) * (int)sizeof(T);
#pragma unroll
      for (int i = 0; i < AW; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            *reinterpret_cast<T*>(base + (32 * i + 8 * (v >> 2) + (v & 3)) * TP + 32 * j * (int)sizeof(T)) =
                (T)(esc * acc[i][j][v]);
    }
    __syncthreads();
#pragma unroll 4
    for (int c = t; c < ROWS * CPR; c += NT) {
      const int r = c / CPR, cc = c % CPR;
      const int m = m0 + hf * ROWS + r;
      if (m >= d.m) continue;
      const char* srcp = tile + r * TP + cc * 16;
      T* dstp = reinterpret_cast<T*>(dst) + (size_t)m * d.n + n0 + cc * PER;
      if (vec) {
        *reinterpret_cast<uint4*>(dstp) = *reinterpret_cast<const uint4*>(srcp);
      } else {
        for (int u = 0; u < PER; ++u)
          if (n0 + cc * PER + u < d.n) dstp[u] = reinterpret_cast<const T*>(srcp)[u];
      }
    }
    if (hf + 1 < HALVES) __syncthreads();
  }
}

template <int FMT, int G, int AW, int NP, int H, bool WIDE>
__device__ __forceinline__ void gemm_body(const GemvDesc& d, int m0, int n0, _Float16* xs, _Float16* ws,
                                          uint8_t* pk, const uint32_t* lut) {
  constexpr int BM = 64 * AW;               // activation rows per tile
  constexpr int XCH = BM * BK / 8 / NT;     // 16-byte activation chunks per thread per step
  constexpr int XBUF = BM * PH, WBUF = BN * PH, PBUF = BN * WP;
  constexpr int SPG = G / BK;               // steps per group
  constexpr int SLOTS = 2 * AW * (BK / 16);  // MFMAs per wave and step
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int mb = (wave >> 1) * 32 * AW, nb = (wave & 1) * 64;
  const int nsteps = d.ng * SPG;
  // this tile's K part: steps [s0, s1), s0 a multiple of WSTEPS
  const int s0 = d.ks0, s1 = d.ks1;
  const int g0 = s0 / SPG, w0 = s0 / WSTEPS;

  f16v_t acc[AW][2];
#pragma unroll
  for (int i = 0; i < AW; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f16v_t{};

  // decoded weight row dr; this thread takes trits [32H, 32H + 32) of each step
  const int dr = t & (BN - 1);
  const uint32_t row = (uint32_t)(n0 + dr);
  Src S;
  const uint32_t n = (uint32_t)d.n, ng = (uint32_t)d.ng, stride = (uint32_t)d.stride;
  S.p0 = rsrc(d.plane0, n * stride);
  S.sc = rsrc(d.scale0, n * ng * 2u);
  S.offg = rsrc(d.offset, d.offset_mode == 2 ? n * ng * 2u : 0u);
  S.sc_v = row * ng * 2u;
  S.offg_v = row * ng * 2u;
  S.mask_v = row * (uint32_t)d.mwords * 4u;
  const uint32_t ro = __builtin_amdgcn_raw_buffer_load_b16(rsrc(d.offset, d.offset_mode == 1 ? n * 2u : 0u), row * 2u, 0, 0);
  Walk<NP> W;
  // NP can exceed this matrix's residual planes (a grouped launch takes the
  // most of its matrices): an absent plane's buffers are NULL and get
  // zero-size resources, so every load from them reads zero (no residual).
  // The walk starts at the part's first group: rowptr plus the mask bits
  // before it.
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const bool on = p < d.planes - 1;
    const uint32_t nnz = on ? (p == 0 ? d.nnz[0] : d.nnz[1]) : 0u;
    S.mask[p] = rsrc(p == 0 ? d.mask[0] : d.mask[1], on ? n * (uint32_t)d.mwords * 4u : 0u);
    S.blk[p] = rsrc(p == 0 ? d.blocks[0] : d.blocks[1], nnz * (uint32_t)(G / 4));
    S.rsc[p] = rsrc(p == 0 ? d.rscale[0] : d.rscale[1], nnz * 2u);
    uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(rsrc(p == 0 ? d.rowptr[0] : d.rowptr[1], on ? n * 4u : 0u),
                                                      row * 4u, 0, 0);
    for (int w = 0; w < (g0 >> 5); ++w) e += __popc(__builtin_amdgcn_raw_buffer_load_b32(S.mask[p], S.mask_v, 4 * w, 0));
    W.mwl[p] = __builtin_amdgcn_raw_buffer_load_b32(S.mask[p], S.mask_v, 4 * (g0 >> 5), 0);
    W.mwn[p] = __builtin_amdgcn_raw_buffer_load_b32(S.mask[p], S.mask_v, 4 * min((g0 >> 5) + 1, d.mwords - 1), 0);
    W.e[p] = e + __popc(W.mwl[p] & ((1u << (g0 & 31)) - 1u));
  }
  // activation chunks (rows past m read as zero) and packed-window chunks
  const __amdgpu_buffer_rsrc_t xr = rsrc(d.x, (uint32_t)d.m * (uint32_t)d.k * 2u);
  uint32_t xo[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = i * NT + t;
    xo[i] = (uint32_t)(m0 + (c >> 3)) * (uint32_t)d.k * 2u + (uint32_t)(c & 7) * 16u;
  }
  // Window chunk i (of WCH) of this thread: row (t >> 2) + 64 i, bytes
  // 16 (t & 3) .. + 16 of the window.  Every offset that can leave the buffer
  // sits in the per-lane offset (rows past n read as zero); windows past the
  // last one reload the last one.
  const uint32_t wo = (uint32_t)(n0 + (t >> 2)) * stride + (uint32_t)(t & 3) * 16u;
  const int wlast = (nsteps - 1) / WSTEPS;
  uint8_t* const wl = pk + (t >> 2) * WP + (t & 3) * 16;
#define TERN_WLOAD(WV_, W_, I_)                                                                   \
  WV_ = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(                         \
      S.p0, wo + (uint32_t)(win_start<FMT>(min((W_), wlast)) + (I_) * 64 * (int)stride), 0, 0))
#define TERN_WSTORE(WV_, W_, I_) \
  *reinterpret_cast<uint4*>(wl + ((W_) % NWIN) * PBUF + (I_) * 64 * WP) = WV_

  // two register sets of prefetched operands: step s uses set s & 1
  uint4 xv0[XCH], xv1[XCH], wv;
  Pre<NP> P0, P1;
  // Products of step s from LDS buffers XB_/WB_ with, between the MFMAs:
  // the loads of step s + 2 (set XL_/PL_, group gl; on even steps one chunk
  // of the window after next), the decode of step s + 1 (D_, written to WS_)
  // and the activation chunks of step s + 1 (XN_, to XS_; on odd steps the
  // window chunk loaded a step ago).  Every step issues the same loads, so
  // the waits the compiler places for them are exact; each MFMA is followed by
  // one piece of this work, which runs on the vector ALU, LDS and the memory
  // pipeline while the matrix core works.  The fragments of the next 16-wide
  // K slice are read while this slice's MFMAs run.
#define TERN_PRODUCTS(U_, XB_, WB_, XL_, PL_, AL_, XN_, XS_, D_, WS_, DN_, PNN_)                  \
  {                                                                                               \
    h8_t fa[2][AW], fb[2][2];                                                                     \
    _Pragma("unroll") for (int i = 0; i < AW; ++i)                                                \
      fa[0][i] = *reinterpret_cast<const h8_t*>(&(XB_)[(mb + 32 * i + (lane & 31)) * PH + 8 * (lane >> 5)]); \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                 \
      fb[0][j] = *reinterpret_cast<const h8_t*>(&(WB_)[(nb + 32 * j + (lane & 31)) * PH + 8 * (lane >> 5)]); \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    _Pragma("unroll") for (int kk = 0; kk < BK / 16; ++kk) {                                      \
      _Pragma("unroll") for (int idx = 0; idx < 2 * AW; ++idx) {                                  \
        acc[idx >> 1][idx & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(                          \
            fa[kk & 1][idx >> 1], fb[kk & 1][idx & 1], acc[idx >> 1][idx & 1], 0, 0, 0);          \
        if (idx == 0 && kk + 1 < BK / 16) {                                                       \
          _Pragma("unroll") for (int i = 0; i < AW; ++i)                                          \
            fa[(kk + 1) & 1][i] = *reinterpret_cast<const h8_t*>(                                 \
                &(XB_)[(mb + 32 * i + (lane & 31)) * PH + 16 * (kk + 1) + 8 * (lane >> 5)]);      \
          _Pragma("unroll") for (int j = 0; j < 2; ++j)                                           \
            fb[(kk + 1) & 1][j] = *reinterpret_cast<const h8_t*>(                                 \
                &(WB_)[(nb + 32 * j + (lane & 31)) * PH + 16 * (kk + 1) + 8 * (lane >> 5)]);      \
        }                                                                                         \
        const int c = kk * 2 * AW + idx; /* slot */                                               \
        if (c == 0) load_step<G, NP, AL_>(S, gl, min(gl, d.ng - 1), W, PL_);                     \
        if (c == 0 && (U_) == 0) {                                                                \
          _Pragma("unroll") for (int p = 0; p < NP; ++p)                                          \
            W.mwn[p] = __builtin_amdgcn_raw_buffer_load_b32(S.mask[p], S.mask_v,                    \
                                                            4 * min((gl >> 5) + 1, d.mwords - 1), 0); \
        }                                                                                         \
        if (c < XCH)                                                                              \
          (XL_)[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(            \
              xr, xo[c], min(s + 2, nsteps - 1) * BK * 2, 0));                                    \
        if (c == XCH && (U_) == 0) TERN_WLOAD(wv, w0 + (q >> 1) + 2, q & 1);                      \
        if (c < 16) (D_).pair(c);                                                                 \
        if (SLOTS > 16) {                                                                         \
          if (c >= 16 && c < 20) (D_).store(c - 16, WS_);                                         \
          if (c >= 20 && c < 20 + XCH) {                                                          \
            const int cx = (c - 20) * NT + t;                                                     \
            *reinterpret_cast<uint4*>(&(XS_)[(cx >> 3) * PH + (cx & 7) * 8]) = (XN_)[c - 20];     \
          }                                                                                       \
          if (c == 20 + XCH && (U_) == 1) TERN_WSTORE(wv, w0 + (q >> 1) + 2, q & 1);              \
        } else if (c == SLOTS - 1) {                                                              \
          _Pragma("unroll") for (int q_ = 0; q_ < 4; ++q_) (D_).store(q_, WS_);                   \
          _Pragma("unroll") for (int i = 0; i < XCH; ++i) {                                       \
            const int cx = i * NT + t;                                                            \
            *reinterpret_cast<uint4*>(&(XS_)[(cx >> 3) * PH + (cx & 7) * 8]) = (XN_)[i];          \
          }                                                                                       \
          if ((U_) == 1) TERN_WSTORE(wv, w0 + (q >> 1) + 2, q & 1);                               \
        }                                                                                         \
        if (c == SLOTS - 1) {                                                                     \
          const int g2 = (s + 2) / SPG, w2 = (s + 2) / WSTEPS;                                    \
          (DN_).prep(g2, (s + 2) & (WSTEPS - 1), win_start<FMT>(w2), pk + (w2 % NWIN) * PBUF + dr * WP, \
                     PNN_, ro, lut);                                                              \
        }                                                                                         \
        __builtin_amdgcn_sched_barrier(0);                                                        \
      }                                                                                           \
    }                                                                                             \
  }
  // Step s = 2q + U_: the products with everything else in their shadow (the
  // decode of step s + 1 was prepared at the end of step s - 1; the last slot
  // prepares step s + 2's), then the barrier that publishes step s + 1's LDS
  // buffers.  Loads past the last step read past the end of
  // x and of the packed rows, which the buffer resources answer with zeros or
  // bytes of the next row; nothing reads what they stage.
#define TERN_STEP(U_, XL_, PL_, XN_, DN_, DL_)                                                    \
  do {                                                                                            \
    const int s = s0 + 2 * q + (U_);                                                              \
    constexpr int AL_ = BK * ((U_) % SPG) + 32 * H;                                               \
    const int gn = (s + 1) / SPG, gl = (s + 2) / SPG;                                             \
    if (gl != gn) walk_next<NP>(gn, W);                                                           \
    TERN_PRODUCTS(U_, xs + (s & 1) * XBUF, ws + (s & 1) * WBUF, XL_, PL_, AL_, XN_,              \
                  xs + ((s + 1) & 1) * XBUF, DN_, ws + ((s + 1) & 1) * WBUF + dr * PH + 32 * H,   \
                  DL_, PL_)                                                                       \
    __syncthreads();                                                                              \
  } while (0)

  // prologue: windows w0 and w0 + 1 and the activation chunks of step s0 to
  // LDS, loads of steps s0 and s0 + 1, decode of step s0
  {
    uint4 w00, w01, w10, w11;
    TERN_WLOAD(w00, w0, 0);
    TERN_WLOAD(w01, w0, 1);
    TERN_WLOAD(w10, w0 + 1, 0);
    TERN_WLOAD(w11, w0 + 1, 1);
    TERN_WSTORE(w00, w0, 0);
    TERN_WSTORE(w01, w0, 1);
    TERN_WSTORE(w10, w0 + 1, 0);
    TERN_WSTORE(w11, w0 + 1, 1);
  }
#pragma unroll
  for (int i = 0; i < XCH; ++i)
    xv0[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo[i], s0 * BK * 2, 0));
  load_step<G, NP, 32 * H>(S, g0, g0, W, P0);
  if (SPG == 1) walk_next<NP>(g0, W);
#pragma unroll
  for (int i = 0; i < XCH; ++i)
    xv1[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo[i], min(s0 + 1, nsteps - 1) * BK * 2, 0));
  load_step<G, NP, (BK % G) + 32 * H>(S, (s0 + 1) / SPG, min((s0 + 1) / SPG, d.ng - 1), W, P1);
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = i * NT + t;
    *reinterpret_cast<uint4*>(&xs[(c >> 3) * PH + (c & 7) * 8]) = xv0[i];
  }
  __syncthreads();
  // decoders by step parity (their K offset within the group differs when a
  // group spans two steps)
  Dec<FMT, G, NP, 32 * H, WIDE> De;
  Dec<FMT, G, NP, (BK % G) + 32 * H, WIDE> Do;
  De.prep(g0, 0, win_start<FMT>(w0), pk + (w0 % NWIN) * PBUF + dr * WP, P0, ro, lut);
#pragma unroll
  for (int i = 0; i < 16; ++i) De.pair(i);
#pragma unroll
  for (int q_ = 0; q_ < 4; ++q_) De.store(q_, &ws[dr * PH + 32 * H]);
  Do.prep((s0 + 1) / SPG, (s0 + 1) & (WSTEPS - 1), win_start<FMT>(w0), pk + (w0 % NWIN) * PBUF + dr * WP, P1, ro,
          lut);
  __syncthreads();
  int q = 0;
  for (; s0 + 2 * q + 1 < s1; ++q) {
    TERN_STEP(0, xv0, P0, xv1, Do, De);
    TERN_STEP(1, xv1, P1, xv0, De, Do);
  }
  if ((s1 - s0) & 1) TERN_STEP(0, xv0, P0, xv1, Do, De);
#undef TERN_STEP
#undef TERN_PRODUCTS
#undef TERN_WSTORE
#undef TERN_WLOAD

  // ---- epilogue: y = 0.5 * acc (the narrow tile held 2 W~; the wide one W~),
  // or the FP32 partial sums of this K part
  constexpr float esc = WIDE ? 1.f : 0.5f;
  if (d.kpart >= 0)
    epilogue<float, AW>(d, m0, n0, acc, reinterpret_cast<char*>(xs), d.partial + (size_t)d.kpart * d.m * d.n, esc);
  else if (d.y_f32) epilogue<float, AW>(d, m0, n0, acc, reinterpret_cast<char*>(xs), d.y, esc);
  else epilogue<_Float16, AW>(d, m0, n0, acc, reinterpret_cast<char*>(xs), d.y, esc);
}

// ---- small M (1..16 activation rows): 16 x 128 output tiles with
// v_mfma_f32_16x16x32_f16, K split into step ranges.  Every weight of a range
// is decoded once; the MFMAs are few, so the decode, not the matrix core,
// sets the pace, and the step loop needs no interleaving.  The loads, the
// LDS windows, the decode and the residual walk are those of the large-tile
// body above.  A workgroup covers steps [s0, s1) (s0 a multiple of WSTEPS);
// with split >= 0 it writes FP32 partial sums to
// d.partial[split][m][n], else y.
typedef float f4v_t __attribute__((ext_vector_type(4)));
constexpr int BMS = 16;  // activation rows of a small tile

template <int FMT, int G, int NP, int H, bool WIDE>
__device__ __forceinline__ void small_body(const GemvDesc& d, int n0, int s0, int s1, int split, _Float16* xs,
                                           _Float16* ws, uint8_t* pk, const uint32_t* lut) {
  constexpr int XBUF = BMS * PH, WBUF = BN * PH, PBUF = BN * WP;
  constexpr int SPG = G / BK;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int nsteps = d.ng * SPG;

  f4v_t acc[2] = {f4v_t{0.f, 0.f, 0.f, 0.f}, f4v_t{0.f, 0.f, 0.f, 0.f}};

  const int dr = t & (BN - 1);
  const uint32_t row = (uint32_t)(n0 + dr);
  Src S;
  const uint32_t n = (uint32_t)d.n, ng = (uint32_t)d.ng, stride = (uint32_t)d.stride;
  S.p0 = rsrc(d.plane0, n * stride);
  S.sc = rsrc(d.scale0, n * ng * 2u);
  S.offg = rsrc(d.offset, d.offset_mode == 2 ? n * ng * 2u : 0u);
  S.sc_v = row * ng * 2u;
  S.offg_v = row * ng * 2u;
  S.mask_v = row * (uint32_t)d.mwords * 4u;
  const uint32_t ro = __builtin_amdgcn_raw_buffer_load_b16(rsrc(d.offset, d.offset_mode == 1 ? n * 2u : 0u), row * 2u, 0, 0);
  // residual walk at the range's first group: rowptr plus the mask bits before it
  const int g0 = s0 / SPG;
  Walk<NP> W;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const bool on = p < d.planes - 1;
    const uint32_t nnz = on ? (p == 0 ? d.nnz[0] : d.nnz[1]) : 0u;
    S.mask[p] = rsrc(p == 0 ? d.mask[0] : d.mask[1], on ? n * (uint32_t)d.mwords * 4u : 0u);
    S.blk[p] = rsrc(p == 0 ? d.blocks[0] : d.blocks[1], nnz * (uint32_t)(G / 4));
    S.rsc[p] = rsrc(p == 0 ? d.rscale[0] : d.rscale[1], nnz * 2u);
    uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(rsrc(p == 0 ? d.rowptr[0] : d.rowptr[1], on ? n * 4u : 0u),
                                                      row * 4u, 0, 0);
    {
      // the mask words before the range's word: the first 8 requested together
      uint32_t mw8[8];
#pragma unroll
      for (int w = 0; w < 8; ++w)
        mw8[w] = __builtin_amdgcn_raw_buffer_load_b32(S.mask[p], w < (g0 >> 5) ? S.mask_v + 4u * w : kOOB, 0, 0);
#pragma unroll
      for (int w = 0; w < 8; ++w) e += __popc(mw8[w]);
      for (int w = 8; w < (g0 >> 5); ++w) e += __popc(__builtin_amdgcn_raw_buffer_load_b32(S.mask[p], S.mask_v, 4 * w, 0));
    }
    W.mwl[p] = __builtin_amdgcn_raw_buffer_load_b32(S.mask[p], S.mask_v, 4 * (g0 >> 5), 0);
    W.mwn[p] = __builtin_amdgcn_raw_buffer_load_b32(S.mask[p], S.mask_v, 4 * min((g0 >> 5) + 1, d.mwords - 1), 0);
    W.e[p] = e + __popc(W.mwl[p] & ((1u << (g0 & 31)) - 1u));
  }
  // activation chunks: threads t < 128 take row t >> 3, chunk t & 7 (rows past m read as zero)
  const __amdgpu_buffer_rsrc_t xr = rsrc(d.x, (uint32_t)d.m * (uint32_t)d.k * 2u);
  const uint32_t xo = t < 128 ? (uint32_t)(t >> 3) * (uint32_t)d.k * 2u + (uint32_t)(t & 7) * 16u : kOOB;
  const uint32_t wo = (uint32_t)(n0 + (t >> 2)) * stride + (uint32_t)(t & 3) * 16u;
  const int w0 = s0 / WSTEPS, wlast = (nsteps - 1) / WSTEPS;
  uint8_t* const wl = pk + (t >> 2) * WP + (t & 3) * 16;
#define TERN_WLOAD(WV_, W_, I_)                                                                   \
  WV_ = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(                         \
      S.p0, wo + (uint32_t)(win_start<FMT>(min((W_), wlast)) + (I_) * 64 * (int)stride), 0, 0))
#define TERN_WSTORE(WV_, W_, I_) \
  *reinterpret_cast<uint4*>(wl + ((W_) % NWIN) * PBUF + (I_) * 64 * WP) = WV_
#define TERN_XLOADS(XV_, S_) \
  XV_ = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo, min((S_), nsteps - 1) * BK * 2, 0))
#define TERN_XSTORES(XV_, BUF_) \
  if (t < 128) *reinterpret_cast<uint4*>(&(BUF_)[(t >> 3) * PH + (t & 7) * 8]) = XV_

  uint4 xv0, xv1, wv;
  Pre<NP> P0, P1;
  // Step s = s0 + 2q + U_ (buffers by relative parity): the per-step loads
  // of step s + 3 (into the set step s + 1 used; its decode was prepared a
  // step ago), the activation tile of step s + 2, the 4 MFMAs of step s, the
  // decode of step s + 1 and its activation chunks to the other buffers, the
  // preparation of step s + 2's decode (from loads issued a step ago),
  // barrier.
#define TERN_SSTEP(U_, XL_, PL_, PP_, XN_, DN_, DL_)                                              \
  do {                                                                                            \
    const int s = s0 + 2 * q + (U_);                                                              \
    constexpr int AL_ = BK * (((U_) + 1) % SPG) + 32 * H;                                         \
    const int g2 = (s + 2) / SPG, gl = (s + 3) / SPG;                                             \
    if (gl != g2) walk_next<NP>(g2, W);                                                           \
    load_step<G, NP, AL_>(S, gl, min(gl, d.ng - 1), W, PL_);                                      \
    if ((U_) == 0) {                                                                              \
      _Pragma("unroll") for (int p = 0; p < NP; ++p)                                              \
        W.mwn[p] = __builtin_amdgcn_raw_buffer_load_b32(S.mask[p], S.mask_v,                      \
                                                        4 * min((gl >> 5) + 1, d.mwords - 1), 0); \
      TERN_WLOAD(wv, w0 + (q >> 1) + 2, q & 1);                                                   \
    }                                                                                             \
    TERN_XLOADS(XL_, s + 2);                                                                      \
    {                                                                                             \
      const _Float16* xb = xs + ((U_) & 1) * XBUF;                                                \
      const _Float16* wb = ws + ((U_) & 1) * WBUF;                                                \
      _Pragma("unroll") for (int kk = 0; kk < BK; kk += 32) {                                     \
        const h8_t a = *reinterpret_cast<const h8_t*>(&xb[(lane & 15) * PH + kk + 8 * (lane >> 4)]); \
        _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                           \
          const h8_t b = *reinterpret_cast<const h8_t*>(                                          \
              &wb[(32 * wave + 16 * j + (lane & 15)) * PH + kk + 8 * (lane >> 4)]);               \
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);                 \
        }                                                                                         \
      }                                                                                           \
    }                                                                                             \
    _Pragma("unroll") for (int i = 0; i < 16; ++i) (DN_).pair(i);                                 \
    _Pragma("unroll") for (int q_ = 0; q_ < 4; ++q_)                                              \
      (DN_).store(q_, ws + (((U_) + 1) & 1) * WBUF + dr * PH + 32 * H);                           \
    TERN_XSTORES(XN_, xs + (((U_) + 1) & 1) * XBUF);                                              \
    if ((U_) == 1) TERN_WSTORE(wv, w0 + (q >> 1) + 2, q & 1);                                     \
    {                                                                                             \
      const int wd2 = (s + 2) / WSTEPS;                                                           \
      (DL_).prep(g2, (s + 2) & (WSTEPS - 1), win_start<FMT>(wd2), pk + (wd2 % NWIN) * PBUF + dr * WP, \
                 PP_, ro, lut);                                                                   \
    }                                                                                             \
    __syncthreads();                                                                              \
  } while (0)

  // prologue: windows w0 and w0 + 1, loads of steps s0 and s0 + 1, decode of s0
  {
    uint4 a0, a1, b0, b1;
    TERN_WLOAD(a0, w0, 0);
    TERN_WLOAD(a1, w0, 1);
    TERN_WLOAD(b0, w0 + 1, 0);
    TERN_WLOAD(b1, w0 + 1, 1);
    TERN_WSTORE(a0, w0, 0);
    TERN_WSTORE(a1, w0, 1);
    TERN_WSTORE(b0, w0 + 1, 0);
    TERN_WSTORE(b1, w0 + 1, 1);
  }
  TERN_XLOADS(xv0, s0);
  load_step<G, NP, 32 * H>(S, g0, min(g0, d.ng - 1), W, P0);
  if (SPG == 1) walk_next<NP>(g0, W);
  TERN_XLOADS(xv1, s0 + 1);
  load_step<G, NP, (BK % G) + 32 * H>(S, (s0 + 1) / SPG, min((s0 + 1) / SPG, d.ng - 1), W, P1);
  TERN_XSTORES(xv0, xs);
  __syncthreads();
  Dec<FMT, G, NP, 32 * H, WIDE> De;
  Dec<FMT, G, NP, (BK % G) + 32 * H, WIDE> Do;
  De.prep(g0, 0, win_start<FMT>(w0), pk + (w0 % NWIN) * PBUF + dr * WP, P0, ro, lut);
#pragma unroll
  for (int i = 0; i < 16; ++i) De.pair(i);
#pragma unroll
  for (int q_ = 0; q_ < 4; ++q_) De.store(q_, &ws[dr * PH + 32 * H]);
  Do.prep((s0 + 1) / SPG, 1, win_start<FMT>(w0), pk + (w0 % NWIN) * PBUF + dr * WP, P1, ro, lut);
  {
    // step s0 + 2's per-step loads, into the set step s0 used
    const int g1 = (s0 + 1) / SPG, g2 = (s0 + 2) / SPG;
    if (g2 != g1) walk_next<NP>(g1, W);
    load_step<G, NP, 32 * H>(S, g2, min(g2, d.ng - 1), W, P0);
  }
  __syncthreads();
  int q = 0;
  for (; s0 + 2 * q + 1 < s1; ++q) {
    TERN_SSTEP(0, xv0, P1, P0, xv1, Do, De);
    TERN_SSTEP(1, xv1, P0, P1, xv0, De, Do);
  }
  if ((s1 - s0) & 1) TERN_SSTEP(0, xv0, P1, P0, xv1, Do, De);
#undef TERN_SSTEP
#undef TERN_XSTORES
#undef TERN_XLOADS
#undef TERN_WSTORE
#undef TERN_WLOAD

  // ---- epilogue: lane l holds rows 4 (l / 16) + v of columns l % 16 of its two tiles
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int nn = n0 + 32 * wave + 16 * j + (lane & 15);
    if (nn >= d.n) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * (lane >> 4) + v;
      if (m >= d.m) continue;
      const float val = (WIDE ? 1.f : 0.5f) * acc[j][v];  // the narrow tile held 2 W~
      if (split >= 0) d.partial[((size_t)split * d.m + m) * d.n + nn] = val;
      else if (d.y_f32) reinterpret_cast<float*>(d.y)[(size_t)m * d.n + nn] = val;
      else reinterpret_cast<_Float16*>(d.y)[(size_t)m * d.n + nn] = (_Float16)val;
    }
  }
}

// Grouped small-M launch: workgroup b computes the 16 x 128 tile at column
// descs[b].tn0 over steps [descs[b].tm0, descs[b].splits) (tm0: first step,
// splits: end step) into partial slice descs[b].gps (or y when gps < 0).
template <int FMT, int G, int NP, bool WIDE>
__global__ __launch_bounds__(NT) void gemm_small_kernel(const GemvDesc* __restrict__ descs) {
  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * BMS * PH + 2 * BN * PH + NWIN * BN * WP / 2];
  __shared__ uint32_t lut[FMT == 1 ? 256 : 1];
  const GemvDesc d = descs[blockIdx.x];
  _Float16* const xs = smem;
  _Float16* const ws = smem + 2 * BMS * PH;
  uint8_t* const pk = reinterpret_cast<uint8_t*>(smem + 2 * BMS * PH + 2 * BN * PH);
  if (FMT == 1) {
    for (int v = threadIdx.x; v < 256; v += NT) lut[v] = v < 243 ? b3_codes(v) : 0u;
  }
  if ((threadIdx.x >> 7) == 0) small_body<FMT, G, NP, 0, WIDE>(d, d.tn0, d.tm0, d.splits, d.gps, xs, ws, pk, lut);
  else small_body<FMT, G, NP, 1, WIDE>(d, d.tn0, d.tm0, d.splits, d.gps, xs, ws, pk, lut);
}

// y[m][n] = sum_s partial[s][m][n] (in split order) for every product of a
// grouped launch: block b reduces 256 outputs of product r with
// r.begin <= b < next product's begin.
__global__ void reduce_grouped_kernel(const RedDesc* __restrict__ rd, int count) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {  // last product whose first block is <= blockIdx.x
    const int mid = (lo + hi + 1) / 2;
    if (rd[mid].begin <= (int)blockIdx.x) lo = mid;
    else hi = mid - 1;
  }
  const RedDesc r = rd[lo];
  const size_t total = (size_t)r.m * r.n;
  const size_t i = (size_t)(blockIdx.x - r.begin) * 256 + threadIdx.x;
  if (i >= total) return;
  float v = 0.f;
  for (int sp = 0; sp < r.splits; ++sp) v += r.partial[(size_t)sp * total + i];
  if (r.y_f32) reinterpret_cast<float*>(r.y)[i] = v;
  else reinterpret_cast<_Float16*>(r.y)[i] = (_Float16)v;
}

// One BM x 128 output tile at (m0, n0) of the product described by d.
template <int FMT, int G, int AW, int NP, bool WIDE>
__device__ __forceinline__ void gemm_tile(const GemvDesc& d, int m0, int n0) {
  constexpr int BM = 64 * AW;
  __shared__ _Float16 xs[2 * BM * PH];
  __shared__ _Float16 ws[2 * BN * PH];
  __shared__ __attribute__((aligned(16))) uint8_t pk[NWIN * BN * WP];
  __shared__ uint32_t lut[FMT == 1 ? 256 : 1];
  if (FMT == 1) {
    for (int v = threadIdx.x; v < 256; v += NT) lut[v] = v < 243 ? b3_codes(v) : 0u;
  }
  // half of each step decoded by this thread (wave-uniform)
  if ((threadIdx.x >> 7) == 0) gemm_body<FMT, G, AW, NP, 0, WIDE>(d, m0, n0, xs, ws, pk, lut);
  else gemm_body<FMT, G, AW, NP, 1, WIDE>(d, m0, n0, xs, ws, pk, lut);
}

// Tiles are numbered with the weight tile fastest and dealt to the XCDs in
// contiguous runs, so the workgroups that run together on one XCD share an
// activation tile, which then stays in that XCD's L2 (the packed weight tiles
// are small and stream from HBM).
template <int FMT, int G, int AW, int NP, bool WIDE>
__global__ __launch_bounds__(NT) void gemm_kernel(GemvDesc d, int mtiles, int ntiles, int per_xcd) {
  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= mtiles * ntiles) return;
  gemm_tile<FMT, G, AW, NP, WIDE>(d, (tile / ntiles) * (64 * AW), (tile % ntiles) * BN);
}

// A grouped launch: workgroup b computes the tile at (descs[b].tm0,
// descs[b].tn0) of the product descs[b] describes (none if its n is 0).
template <int FMT, int G, int AW, int NP, bool WIDE>
__global__ __launch_bounds__(NT) void gemm_grouped_kernel(const GemvDesc* __restrict__ descs) {
  const GemvDesc d = descs[blockIdx.x];
  if (d.n <= 0) return;  // a position left open by the XCD layout
  gemm_tile<FMT, G, AW, NP, WIDE>(d, d.tm0, d.tn0);
}

__global__ void zero_fill_kernel(void* y, size_t count, int f32) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  if (f32) reinterpret_cast<float*>(y)[i] = 0.f;
  else reinterpret_cast<uint16_t*>(y)[i] = 0;
}

}  // namespace

bool gemm_wide(int np, bool offsets) { return np >= 2 || (np == 1 && offsets); }

hipError_t launch_gemm(const GemvDesc& d, int format, hipStream_t s) {
  if (d.m <= 0 || d.n <= 0) return hipSuccess;
  if (d.ng == 0) {
    const size_t count = (size_t)d.m * d.n;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, d.y, count, d.y_f32);
    return hipGetLastError();
  }
  if (!(format == 0 || format == 1) || !(d.group == 64 || d.group == 128)) return hipErrorInvalidValue;
  // 256-row activation tiles once M fills them; 128-row tiles below
  const int aw = gemm_tile_rows(d.m) / 64;
  const int mtiles = (d.m + 64 * aw - 1) / (64 * aw), ntiles = (d.n + BN - 1) / BN;
  const int per_xcd = (mtiles * ntiles + 7) / 8;
  const dim3 grid(8 * per_xcd);
  const bool wide = gemm_wide(d.planes - 1, d.offset_mode != 0);
#define TERN_GEMM_LAUNCH(F, G_, AW_, NP_, W_) \
  hipLaunchKernelGGL((gemm_kernel<F, G_, AW_, NP_, W_>), grid, dim3(NT), 0, s, d, mtiles, ntiles, per_xcd)
#define TERN_GEMM_NP(F, G_, AW_)                                          \
  do {                                                                    \
    if (d.planes == 1) TERN_GEMM_LAUNCH(F, G_, AW_, 0, false);            \
    else if (d.planes == 2 && !wide) TERN_GEMM_LAUNCH(F, G_, AW_, 1, false); \
    else if (d.planes == 2) TERN_GEMM_LAUNCH(F, G_, AW_, 1, true);        \
    else TERN_GEMM_LAUNCH(F, G_, AW_, 2, true);                           \
  } while (0)
  if (format == 0) {
    if (d.group == 64) { if (aw == 4) TERN_GEMM_NP(0, 64, 4); else TERN_GEMM_NP(0, 64, 2); }
    else { if (aw == 4) TERN_GEMM_NP(0, 128, 4); else TERN_GEMM_NP(0, 128, 2); }
  } else {
    if (d.group == 64) { if (aw == 4) TERN_GEMM_NP(1, 64, 4); else TERN_GEMM_NP(1, 64, 2); }
    else { if (aw == 4) TERN_GEMM_NP(1, 128, 4); else TERN_GEMM_NP(1, 128, 2); }
  }
#undef TERN_GEMM_NP
#undef TERN_GEMM_LAUNCH
  return hipGetLastError();
}

int gemm_wgs_per_cu(int format, int aw) {
  // the static LDS of gemm_tile: activation and decoded-weight double
  // buffers, packed windows and (base-3) the code table; 160 KB per CU
  const size_t bm = 64 * (size_t)aw;
  const size_t lds = 2 * bm * PH * 2 + 2 * (size_t)BN * PH * 2 + (size_t)NWIN * BN * WP + (format == 1 ? 1024 : 4);
  return std::max(1, (int)((160u * 1024u) / lds));
}

hipError_t launch_gemm_grouped(const GemvDesc* descs, int count, int format, int group, int aw, int np,
                               bool offsets, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (!(format == 0 || format == 1) || !(group == 64 || group == 128) || !(aw == 2 || aw == 4) || np < 0 || np > 2)
    return hipErrorInvalidValue;
  const dim3 grid(count);
  const bool wide = gemm_wide(np, offsets);
#define TERN_GG(F, G_, AW_, NP_, W_) \
  hipLaunchKernelGGL((gemm_grouped_kernel<F, G_, AW_, NP_, W_>), grid, dim3(NT), 0, s, descs)
#define TERN_GG_NP(F, G_, AW_)                              \
  do {                                                      \
    if (np == 0) TERN_GG(F, G_, AW_, 0, false);             \
    else if (np == 1 && !wide) TERN_GG(F, G_, AW_, 1, false); \
    else if (np == 1) TERN_GG(F, G_, AW_, 1, true);         \
    else TERN_GG(F, G_, AW_, 2, true);                      \
  } while (0)
  if (format == 0) {
    if (group == 64) { if (aw == 4) TERN_GG_NP(0, 64, 4); else TERN_GG_NP(0, 64, 2); }
    else { if (aw == 4) TERN_GG_NP(0, 128, 4); else TERN_GG_NP(0, 128, 2); }
  } else {
    if (group == 64) { if (aw == 4) TERN_GG_NP(1, 64, 4); else TERN_GG_NP(1, 64, 2); }
    else { if (aw == 4) TERN_GG_NP(1, 128, 4); else TERN_GG_NP(1, 128, 2); }
  }
#undef TERN_GG_NP
#undef TERN_GG
  return hipGetLastError();
}

hipError_t launch_gemm_small(const GemvDesc* descs, int count, int format, int group, int np, bool offsets,
                             hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (!(format == 0 || format == 1) || !(group == 64 || group == 128) || np < 0 || np > 2) return hipErrorInvalidValue;
  const dim3 grid(count);
  const bool wide = gemm_wide(np, offsets);
#define TERN_GS(F, G_, NP_, W_) hipLaunchKernelGGL((gemm_small_kernel<F, G_, NP_, W_>), grid, dim3(NT), 0, s, descs)
#define TERN_GS_NP(F, G_)                             \
  do {                                                \
    if (np == 0) TERN_GS(F, G_, 0, false);            \
    else if (np == 1 && !wide) TERN_GS(F, G_, 1, false); \
    else if (np == 1) TERN_GS(F, G_, 1, true);        \
    else TERN_GS(F, G_, 2, true);                     \
  } while (0)
  if (format == 0) { if (group == 64) TERN_GS_NP(0, 64); else TERN_GS_NP(0, 128); }
  else { if (group == 64) TERN_GS_NP(1, 64); else TERN_GS_NP(1, 128); }
#undef TERN_GS_NP
#undef TERN_GS
  return hipGetLastError();
}

// One thread per tile (plus the reduce entries): the table that a batch
// would copy from host memory, written on the device from SmallSpec.
__global__ void small_tiles_kernel(SmallSpec sp, GemvDesc* __restrict__ tiles, RedDesc* __restrict__ red) {
  const int t = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int per_chunk = sp.nsplit * sp.ntn;
  if (t < sp.nred) red[t] = t == 0 ? sp.red[0] : sp.red[1];
  if (t >= sp.nchunk * per_chunk) return;
  const int c = t / per_chunk, r = t % per_chunk, split = r / sp.ntn;
  GemvDesc d = c == 0 ? sp.base[0] : sp.base[1];
  d.tn0 = (r % sp.ntn) * 128;
  d.tm0 = sp.rg[split];
  d.splits = sp.rg[split + 1];
  d.gps = sp.nsplit > 1 ? split : -1;
  tiles[t] = d;
}

hipError_t launch_small_tiles(const SmallSpec& sp, GemvDesc* tiles, RedDesc* red, hipStream_t s) {
  const int n = std::max(sp.nchunk * sp.nsplit * sp.ntn, sp.nred);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(small_tiles_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, sp, tiles, red);
  return hipGetLastError();
}

hipError_t launch_reduce_grouped(const RedDesc* rd, int count, int blocks, hipStream_t s) {
  if (count <= 0 || blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_grouped_kernel, dim3(blocks), dim3(256), 0, s, rd, count);
  return hipGetLastError();
}

}  // namespace tern
