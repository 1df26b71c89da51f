// Batched product y = x W^T for many activation rows (tuned for M >= 64):
// the packed weights of one group are decoded into an FP16 tile in LDS
// (W~[n,k] = off + s0*t0 + m1*s1*t1 + m2*s2*t2), and the tile product runs on
// the matrix cores (v_mfma_f32_16x16x32_f16, FP32 accumulation).  This is
// the batched-execution direction named by arXiv 2609.09240 (kernel
// optimisation across shapes and batch sizes); at M >= 64 the product is a
// dense contraction, so MFMA is the right unit.
//
// Tile: 128 activation rows x 128 weight rows x one group (BK = G) per step;
// 256 threads = 4 waves in a 2 x 2 arrangement, each wave owning a 64 x 64
// output block of 4 x 4 MFMA tiles.  Operand layout of the 16x16x32 f16 MFMA:
// lane l supplies A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16] and
// receives D[4*(l/16) + v][l%16], v = 0..3.
#include "internal.h"

namespace tern {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, NT = 256;

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// FP16 pair (2*t[2i], 2*t[2i+1]) of 2-bit word w (see the decode kernel).
__device__ __forceinline__ uint32_t pair_of(uint32_t w, int shift) { return (w << shift) & 0xC000C000u; }

__device__ __forceinline__ uint32_t pk_mul(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, a) * __builtin_bit_cast(h2_t, b));
}
__device__ __forceinline__ uint32_t pk_fma(uint32_t a, uint32_t b, uint32_t c) {
  const h2_t r = __builtin_bit_cast(h2_t, a) * __builtin_bit_cast(h2_t, b) + __builtin_bit_cast(h2_t, c);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t splat(uint16_t h) { return (uint32_t)h * 0x10001u; }

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

// Writes FP16 values 2*W~[row, g*G + H*G/2 + i], i < G/2, to dst (LDS).
template <int FMT, int G, int H>
__device__ __forceinline__ void decode_half(const GemvDesc& d, int g, int wrow, bool ok,
                                            const uint32_t* lut, _Float16* dst_h) {
  constexpr int HT = G / 2;  // trits per thread
  uint32_t out[HT / 2];      // FP16 pairs, natural order
#pragma unroll
  for (int i = 0; i < HT / 2; ++i) out[i] = 0u;
  if (ok) {
    const uint8_t* prow = d.plane0 + (size_t)wrow * d.stride;
    const uint32_t s0 = splat(d.scale0[(size_t)wrow * d.ng + g]);
    if (FMT == 0) {
      const uint4* wp = reinterpret_cast<const uint4*>(prow + (size_t)g * (G / 4) + H * (G / 8));
#pragma unroll
      for (int q = 0; q < HT / 64; ++q) {
        const uint4 v = wp[q];
        const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) out[q * 32 + u * 8 + i] = pk_mul(pair_of(ws[u], 14 - 2 * i), s0);
      }
      if (HT % 64) {  // G = 64: 32 trits = two words
        const uint32_t* wq = reinterpret_cast<const uint32_t*>(prow + (size_t)g * (G / 4) + H * (G / 8));
#pragma unroll
        for (int u = 0; u < (HT % 64) / 16; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) out[(HT / 64) * 32 + u * 8 + i] = pk_mul(pair_of(wq[(HT / 64) * 4 + u], 14 - 2 * i), s0);
      }
    } else {
      constexpr int GB = (G + 4) / 5;
      constexpr int B0 = (H * HT) / 5, B1 = (H * HT + HT - 1) / 5, NB = B1 - B0 + 1;
      const uint8_t* gp = prow + (size_t)g * GB;
      uint32_t cw[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) cw[j] = lut[gp[B0 + j]];
#pragma unroll
      for (int i = 0; i < HT / 2; ++i) {
        const int ta = H * HT + 2 * i, tb = ta + 1;
        const uint32_t ca = (cw[ta / 5 - B0] >> (2 * (ta % 5))) & 3u;
        const uint32_t cb = (cw[tb / 5 - B0] >> (2 * (tb % 5))) & 3u;
        out[i] = pk_mul((ca << 14) | (cb << 30), s0);
      }
    }
    for (int p = 0; p < d.planes - 1; ++p) {
      const uint32_t* rm = d.mask[p] + (size_t)wrow * d.mwords;
      if ((rm[g >> 5] >> (g & 31)) & 1u) {
        uint32_t b = d.rowptr[p][wrow];
        for (int w = 0; w < (g >> 5); ++w) b += __popc(rm[w]);
        if (g & 31) b += __popc(rm[g >> 5] & ((1u << (g & 31)) - 1u));
        const uint32_t s1 = splat(d.rscale[p][b]);
        const uint32_t* bp = reinterpret_cast<const uint32_t*>(d.blocks[p] + (size_t)b * (G / 4) + H * (G / 8));
#pragma unroll
        for (int q = 0; q < HT / 16; ++q) {
          const uint32_t w = bp[q];
#pragma unroll
          for (int i = 0; i < 8; ++i) out[q * 8 + i] = pk_fma(pair_of(w, 14 - 2 * i), s1, out[q * 8 + i]);
        }
      }
    }
    if (d.offset_mode != 0) {
      const uint16_t o = d.offset_mode == 1 ? d.offset[wrow] : d.offset[(size_t)wrow * d.ng + g];
      const h2_t ov = __builtin_bit_cast(h2_t, splat(o)) * (h2_t){(_Float16)2.0f, (_Float16)2.0f};
#pragma unroll
      for (int i = 0; i < HT / 2; ++i)
        out[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, out[i]) + ov);
    }
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(dst_h);
#pragma unroll
  for (int i = 0; i < HT / 2; i += 4)
    *reinterpret_cast<uint4*>(dst + i) = make_uint4(out[i], out[i + 1], out[i + 2], out[i + 3]);
}

template <int FMT, int G>
__global__ __launch_bounds__(NT) void gemm_kernel(GemvDesc d) {
  constexpr int BK = G;
  constexpr int XP = BK + 8;  // LDS row pitch in halves (16-byte pad)
  __shared__ _Float16 xs[BM * XP];
  __shared__ _Float16 wt[BN * XP];
  __shared__ uint32_t lut[256];

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;

  if (FMT == 1) {
    for (int v = t; v < 256; v += NT) lut[v] = v < 243 ? b3_codes(v) : 0u;
  }

  f4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

  // decode assignment: thread -> weight row r = t % 128, half h = t / 128 of
  // the group (h is wave-uniform, so the byte indices below are constants)
  const int dr = t & (BN - 1), dh = t >> 7;
  const int wrow = n0 + dr;
  const bool wrow_ok = wrow < d.n;

  for (int g = 0; g < d.ng; ++g) {
    __syncthreads();
    // ---- activation tile: BM x BK halves, 16-byte chunks
#pragma unroll
    for (int i = 0; i < BM * BK / 8 / NT; ++i) {
      const int c = i * NT + t;
      const int r = c / (BK / 8), c8 = c % (BK / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + r < d.m)
        v = *reinterpret_cast<const uint4*>(d.x + (size_t)(m0 + r) * d.k + (size_t)g * BK + c8 * 8);
      *reinterpret_cast<uint4*>(&xs[r * XP + c8 * 8]) = v;
    }
    // ---- weight tile: FP16 values of 2*W~ (the 0.5 is applied in the epilogue)
    if (dh == 0)
      decode_half<FMT, G, 0>(d, g, wrow, wrow_ok, lut, &wt[dr * XP]);
    else
      decode_half<FMT, G, 1>(d, g, wrow, wrow_ok, lut, &wt[dr * XP + G / 2]);
    __syncthreads();
    // ---- MFMA over the group
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      h8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + (lane & 15);
        a[i] = *reinterpret_cast<const h8_t*>(&xs[r * XP + kk + 8 * (lane >> 4)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + (lane & 15);
        b[j] = *reinterpret_cast<const h8_t*>(&wt[r * XP + kk + 8 * (lane >> 4)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + v;
        if (m < d.m && n < d.n) {
          if (d.y_f32)
            reinterpret_cast<float*>(d.y)[(size_t)m * d.n + n] = 0.5f * acc[i][j][v];
          else
            reinterpret_cast<_Float16*>(d.y)[(size_t)m * d.n + n] = (_Float16)(0.5f * acc[i][j][v]);
        }
      }
    }
  }
}

__global__ void zero_fill_kernel(void* y, size_t count, int f32) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  if (f32) reinterpret_cast<float*>(y)[i] = 0.f;
  else reinterpret_cast<uint16_t*>(y)[i] = 0;
}

}  // namespace

hipError_t launch_gemm(const GemvDesc& d, int format, hipStream_t s) {
  if (d.m <= 0 || d.n <= 0) return hipSuccess;
  if (d.ng == 0) {
    const size_t count = (size_t)d.m * d.n;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, d.y, count, d.y_f32);
    return hipGetLastError();
  }
  const dim3 grid((d.n + BN - 1) / BN, (d.m + BM - 1) / BM);
  if (format == 0 && d.group == 64) hipLaunchKernelGGL((gemm_kernel<0, 64>), grid, dim3(NT), 0, s, d);
  else if (format == 0 && d.group == 128) hipLaunchKernelGGL((gemm_kernel<0, 128>), grid, dim3(NT), 0, s, d);
  else if (format == 1 && d.group == 64) hipLaunchKernelGGL((gemm_kernel<1, 64>), grid, dim3(NT), 0, s, d);
  else if (format == 1 && d.group == 128) hipLaunchKernelGGL((gemm_kernel<1, 128>), grid, dim3(NT), 0, s, d);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tern
