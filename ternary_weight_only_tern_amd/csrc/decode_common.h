// Decode-kernel helpers shared by the lane-per-row products (gemv.hip) and the
// base-3 matrix-core decode (gemv_b3.hip): FP16 pair arithmetic, the 2-bit
// pair decode, the wavefront hand-off, and the compacted residual planes.
// Everything sits in an unnamed namespace: each kernel source gets its own
// copy.
#pragma once

#include "internal.h"

#define GLOBAL __attribute__((address_space(1)))

namespace tern {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ const GLOBAL T* gp(const T* p) { return (const GLOBAL T*)p; }

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w), __builtin_bit_cast(h2_t, x), c, false);
}

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ uint32_t pair_of(uint32_t w, int shift) {
  return (w << shift) & 0xC000C000u;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ void wave_sync() {
  // One wavefront's LDS accesses are processed in order; this keeps the
  // compiler from moving LDS accesses across the hand-off between lanes.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Residual plane p, groups [ra, rz) of the 64 rows of this wave, processed
// compacted through the wave's LDS area `buf` (`cap` bytes).
template <int G, int MT>
__device__ __forceinline__ void residual_compact(const GemvDesc& d, int p, int row, bool row_ok,
                                                 int ra, int rz, const GLOBAL uint32_t* const (&xr)[MT],
                                                 uint8_t* buf, int cap, float (&acc)[MT]) {
  const int lane = threadIdx.x % kWave;
  // this row's blocks in [ra, rz): count, first block index
  uint32_t cnt = 0, base = 0;
  const GLOBAL uint32_t* rm = gp(d.mask[p]) + (size_t)(row_ok ? row : 0) * d.mwords;
  if (row_ok) {
    base = gp(d.rowptr[p])[row];
    for (int w = 0; w < (ra >> 5); ++w) base += __popc(rm[w]);
    if (ra & 31) base += __popc(rm[ra >> 5] & ((1u << (ra & 31)) - 1u));
    for (int w = ra >> 5; w <= ((rz - 1) >> 5); ++w) {
      const int lo = max(ra - (w << 5), 0), hi = min(rz - (w << 5), 32);
      const uint32_t keep = (lo > 0 ? ~((1u << lo) - 1u) : ~0u) & (hi < 32 ? ((1u << hi) - 1u) : ~0u);
      cnt += __popc(rm[w] & keep);
    }
  }
  // exclusive prefix of the counts over the wave
  uint32_t incl = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  const uint32_t off = incl - cnt;
  const uint32_t total = __shfl(incl, kWave - 1, kWave);
  if (total == 0) return;

  // window of entries held in LDS: [block index, (row lane << 16) | group], then MT values
  constexpr int ESZ = 8 + 4 * MT;
  const int win = (cap / ESZ) / kWave * kWave;
  uint32_t* ent = reinterpret_cast<uint32_t*>(buf);
  float* val = reinterpret_cast<float*>(buf + (size_t)win * 8);
  const GLOBAL uint8_t* blocks = gp(d.blocks[p]);
  const GLOBAL uint16_t* rscale = gp(d.rscale[p]);

  for (uint32_t w0 = 0; w0 < total; w0 += win) {
    const uint32_t wn = min((uint32_t)win, total - w0);
    wave_sync();
    // each lane lists its own entries that fall in this window
    if (cnt && off < w0 + wn && off + cnt > w0) {
      uint32_t e = off;
      for (int w = ra >> 5; w <= ((rz - 1) >> 5); ++w) {
        const int lo = max(ra - (w << 5), 0), hi = min(rz - (w << 5), 32);
        uint32_t bits = rm[w] & (lo > 0 ? ~((1u << lo) - 1u) : ~0u) & (hi < 32 ? ((1u << hi) - 1u) : ~0u);
        while (bits) {
          const int g = (w << 5) + __builtin_ctz(bits);
          bits &= bits - 1u;
          if (e >= w0 && e < w0 + wn) {
            ent[2 * (e - w0)] = base + (e - off);
            ent[2 * (e - w0) + 1] = ((uint32_t)lane << 16) | (uint32_t)g;
          }
          ++e;
        }
      }
    }
    wave_sync();
    // one lane per block
    for (uint32_t t = lane; t < wn; t += kWave) {
      const uint32_t b = ent[2 * t];
      const int g = (int)(ent[2 * t + 1] & 0xFFFFu);
      const GLOBAL u4_t* blk = reinterpret_cast<const GLOBAL u4_t*>(blocks + (size_t)b * (G / 4));
      float part[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) part[m] = 0.f;
#pragma unroll
      for (int q = 0; q < G / 64; ++q) {
        const u4_t v = __builtin_nontemporal_load(blk + q);
        const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int xd = g * (G / 2) + q * 32 + u * 8;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const GLOBAL u4_t* xv = reinterpret_cast<const GLOBAL u4_t*>(xr[m] + xd);
            const u4_t x0 = xv[0], x1 = xv[1];
            const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) part[m] = dot2(pair_of(ws[u], 14 - 2 * i), xs[i], part[m]);
          }
        }
      }
      const float rs = 0.5f * h2f(rscale[b]);
#pragma unroll
      for (int m = 0; m < MT; ++m) val[t * MT + m] = rs * part[m];
    }
    wave_sync();
    // each lane adds the values of its own entries, in order
    if (cnt) {
      const uint32_t lo = max(off, w0), hi = min(off + cnt, w0 + wn);
      for (uint32_t e = lo; e < hi; ++e)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] += val[(e - w0) * MT + m];
    }
  }
}

}  // namespace
}  // namespace tern
