// Decode-path product y = x W^T for a few activation rows (M <= 8 per pass)
// on packed ternary planes: the direct ternary product ("Can ternary LLMs hit
// 1.58 bits per weight", How It Works: matrix products become additions and
// subtractions; arXiv 2609.09240: the packed weights are consumed directly).
//
// Work item = 64 output rows x one K split; one wavefront per work item, one
// row per lane.  Packed rows are staged through LDS with coalesced 16-byte
// loads (8 or 13 lanes cover 128 or 208 contiguous bytes of a row), then each
// lane decodes its own row.  All lanes sit at the same K position, so the
// activations are wave-uniform and live in SGPRs (scalar loads), which leaves
// the VALU for decode and multiply-accumulate only.
//
// Decode.  A 2-bit word holds 16 trits, even offsets in the low half-word and
// odd offsets in the high half-word, each as a 2-bit two's-complement code.
// Shifting pair i to bits 14..15 / 30..31 and masking with 0xC000C000 gives
// the FP16 pair (2*t[2i], 2*t[2i+1]) exactly (bit 15 = sign, bit 14 = the top
// exponent bit: 0x4000 = 2.0), so one v_dot2_f32_f16 against the natural
// activation pair (x[2i], x[2i+1]) accumulates 2*(t.x) in FP32.  Base-3 bytes
// are first mapped through a 256-entry LDS table to the same 2-bit codes
// (two tables place the five trits of the first / second byte of a pair).
// Per group the FP32 partial is scaled by 0.5*s (exact) and added to the row
// accumulator.  Residual planes are walked per lane over the row's compact
// blocks (divergent loop), and offsets add off * sum(x) per group.
#include "internal.h"

namespace tern {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

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

template <int FMT, int G>
struct Geo {
  static constexpr int GB = FMT == 0 ? G / 4 : (G + 4) / 5;   // bytes per group
  static constexpr int SGB = FMT == 0 ? 128 : 208;             // bytes per row per stage
  static constexpr int SG = SGB / GB;                           // groups per stage
  static constexpr int CPR = SGB / 16;                          // 16-byte chunks per row
  static constexpr int PITCH = FMT == 0 ? 144 : 208;            // LDS row pitch (bytes)
  static constexpr int CHUNKS = kGemvRows * CPR / kWave;        // chunks per lane per stage
  static_assert(SG * GB == SGB, "stage must hold whole groups");
  static_assert((PITCH / 16) % 2 == 1, "odd 16-byte pitch keeps b128 reads conflict-free");
};

// Base-3 byte -> 2-bit codes.  For a byte pair (A, B) holding trits t0..t4 and
// t5..t9, pair i = (t[2i], t[2i+1]) must sit at bits 6+2i (low) and 22+2i
// (high) of lutA[A] | lutB[B]; then pair i decodes with shift 8-2i.
__device__ void build_b3_luts(uint32_t* lutA, uint32_t* lutB) {
  for (int v = threadIdx.x; v < 256; v += kWave) {
    uint32_t a = 0, b = 0;
    if (v < 243) {
      int r = v;
      uint32_t c[5];
      for (int i = 0; i < 5; ++i) {
        c[i] = (uint32_t)((r % 3) - 1) & 3u;
        r /= 3;
      }
      // first byte of a pair: t0 t1 t2 t3 t4 -> pair0 lo/hi, pair1 lo/hi, pair2 lo
      a = (c[0] << 6) | (c[1] << 22) | (c[2] << 8) | (c[3] << 24) | (c[4] << 10);
      // second byte: t5 t6 t7 t8 t9 -> pair2 hi, pair3 lo/hi, pair4 lo/hi
      b = (c[0] << 26) | (c[1] << 12) | (c[2] << 28) | (c[3] << 14) | (c[4] << 30);
    }
    lutA[v] = a;
    lutB[v] = b;
  }
}

__device__ __forceinline__ int find_desc(const GemvDesc* descs, int ndesc, int item) {
  int lo = 0, hi = ndesc - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (descs[mid].tile_begin <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Multiply-accumulate the 2-bit word w (16 trits starting at activation
// dword xd) against MT activation rows.
template <int MT>
__device__ __forceinline__ void mac_word(uint32_t w, const uint32_t* const (&xr)[MT], int xd,
                                         float (&acc)[MT]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t p = pair_of(w, 14 - 2 * i);
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = dot2(p, xr[m][xd + i], acc[m]);
  }
}

template <int FMT, int G, int MT>
__global__ __launch_bounds__(kWave) void gemv_kernel(const GemvDesc* __restrict__ descs, int ndesc,
                                                     GemvDesc one) {
  using Gm = Geo<FMT, G>;
  extern __shared__ uint4 stage[];  // [64 rows][PITCH bytes]
  __shared__ uint32_t lutA[FMT == 1 ? 256 : 1];
  __shared__ uint32_t lutB[FMT == 1 ? 256 : 1];

  const int item_g = blockIdx.x;
  const GemvDesc& d = ndesc ? descs[find_desc(descs, ndesc, item_g)] : one;
  const int item = item_g - d.tile_begin;
  const int rb = item % d.row_blocks;
  const int split = item / d.row_blocks;
  const int lane = threadIdx.x;
  const int row = rb * kGemvRows + lane;
  const bool row_ok = row < d.n;
  const int g0 = split * d.gps;
  const int g1 = min(d.ng, g0 + d.gps);
  const int nstages = (g1 - g0 + Gm::SG - 1) / Gm::SG;

  if (FMT == 1) {
    build_b3_luts(lutA, lutB);
  }

  const uint32_t* xr[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
    xr[m] = reinterpret_cast<const uint32_t*>(d.x + (size_t)min(m, d.m - 1) * d.k);

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;

  const uint8_t* prow0 = d.plane0 + (size_t)rb * kGemvRows * d.stride;
  const int rows_here = min(kGemvRows, d.n - rb * kGemvRows);
  uint8_t* lds = reinterpret_cast<uint8_t*>(stage);

  uint4 pre[Gm::CHUNKS];
  uint16_t spre[Gm::SG];
  auto load_stage = [&](int s) {
    const int gs = g0 + s * Gm::SG;
    const int bytes = min(Gm::SG, g1 - gs) * Gm::GB;
    const uint8_t* base = prow0 + (size_t)gs * Gm::GB;
#pragma unroll
    for (int i = 0; i < Gm::CHUNKS; ++i) {
      const int c = i * kWave + lane;
      const int r = c / Gm::CPR, col = c % Gm::CPR;
      if (r < rows_here && col * 16 < bytes)
        pre[i] = *reinterpret_cast<const uint4*>(base + (size_t)r * d.stride + col * 16);
    }
#pragma unroll
    for (int j = 0; j < Gm::SG; ++j)
      spre[j] = (row_ok && gs + j < g1) ? d.scale0[(size_t)row * d.ng + gs + j] : (uint16_t)0;
  };

  if (nstages > 0) load_stage(0);
  for (int s = 0; s < nstages; ++s) {
    const int gs = g0 + s * Gm::SG;
    const int ngs = min(Gm::SG, g1 - gs);
    __syncthreads();  // previous stage fully consumed (and LUTs built)
#pragma unroll
    for (int i = 0; i < Gm::CHUNKS; ++i) {
      const int c = i * kWave + lane;
      const int r = c / Gm::CPR, col = c % Gm::CPR;
      *reinterpret_cast<uint4*>(lds + r * Gm::PITCH + col * 16) = pre[i];
    }
    float sc[Gm::SG];
#pragma unroll
    for (int j = 0; j < Gm::SG; ++j) sc[j] = 0.5f * h2f(spre[j]);
    __syncthreads();
    if (s + 1 < nstages) load_stage(s + 1);

    const uint8_t* my = lds + lane * Gm::PITCH;
#pragma unroll
    for (int j = 0; j < Gm::SG; ++j) {
      if (j < ngs) {
        const int g = gs + j;
        const int xg = g * (G / 2);  // activation dword index of the group start
        float part[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) part[m] = 0.f;
        if (FMT == 0) {
#pragma unroll
          for (int q = 0; q < G / 64; ++q) {
            const uint4 v = *reinterpret_cast<const uint4*>(my + j * Gm::GB + q * 16);
            mac_word<MT>(v.x, xr, xg + q * 32 + 0, part);
            mac_word<MT>(v.y, xr, xg + q * 32 + 8, part);
            mac_word<MT>(v.z, xr, xg + q * 32 + 16, part);
            mac_word<MT>(v.w, xr, xg + q * 32 + 24, part);
          }
        } else {
          constexpr int GB = Gm::GB;
          const int off = j * GB;               // compile-time after unrolling
          const int c0 = off >> 4;
          uint32_t dw[12];
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            if (((off + GB - 1) >> 4) >= c0 + q) {
              const uint4 v = *reinterpret_cast<const uint4*>(my + (c0 + q) * 16);
              dw[4 * q + 0] = v.x; dw[4 * q + 1] = v.y; dw[4 * q + 2] = v.z; dw[4 * q + 3] = v.w;
            } else {
              dw[4 * q + 0] = dw[4 * q + 1] = dw[4 * q + 2] = dw[4 * q + 3] = 0u;
            }
          }
          const int sh = off - c0 * 16;
#pragma unroll
          for (int bp = 0; bp < (GB + 1) / 2; ++bp) {
            const int ia = sh + 2 * bp, ib = ia + 1;
            const uint32_t ba = (dw[ia >> 2] >> ((ia & 3) * 8)) & 0xFFu;
            uint32_t code = lutA[ba];
            if (2 * bp + 1 < GB) {
              const uint32_t bb = (dw[ib >> 2] >> ((ib & 3) * 8)) & 0xFFu;
              code |= lutB[bb];
            }
#pragma unroll
            for (int i = 0; i < 5; ++i) {
              if (10 * bp + 2 * i < G) {
                const uint32_t p = pair_of(code, 8 - 2 * i);
#pragma unroll
                for (int m = 0; m < MT; ++m) part[m] = dot2(p, xr[m][xg + 5 * bp + i], part[m]);
              }
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = fmaf(sc[j], part[m], acc[m]);
      }
    }
  }

  // ---- residual planes: each lane walks its row's compact blocks in [g0, g1)
  if (d.planes > 1 && row_ok) {
    for (int p = 0; p < d.planes - 1; ++p) {
      const uint32_t* rm = d.mask[p] + (size_t)row * d.mwords;
      uint32_t b = d.rowptr[p][row];
      for (int w = 0; w < (g0 >> 5); ++w) b += __popc(rm[w]);
      if (g0 & 31) b += __popc(rm[g0 >> 5] & ((1u << (g0 & 31)) - 1u));
      for (int w = g0 >> 5; w <= ((g1 - 1) >> 5) && g1 > g0; ++w) {
        uint32_t bits = rm[w];
        const int lo = max(g0 - (w << 5), 0), hi = min(g1 - (w << 5), 32);
        bits &= (lo > 0 ? ~((1u << lo) - 1u) : ~0u) & (hi < 32 ? ((1u << hi) - 1u) : ~0u);
        while (bits) {
          const int g = (w << 5) + __builtin_ctz(bits);
          bits &= bits - 1u;
          const uint4* blk = reinterpret_cast<const uint4*>(d.blocks[p] + (size_t)b * (G / 4));
          float part[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) part[m] = 0.f;
#pragma unroll
          for (int q = 0; q < G / 64; ++q) {
            const uint4 v = blk[q];
            const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int xd = g * (G / 2) + q * 32 + u * 8;
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const uint32_t pr = pair_of(ws[u], 14 - 2 * i);
#pragma unroll
                for (int m = 0; m < MT; ++m) part[m] = dot2(pr, xr[m][xd + i], part[m]);
              }
            }
          }
          const float rs = 0.5f * h2f(d.rscale[p][b]);
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[m] = fmaf(rs, part[m], acc[m]);
          ++b;
        }
      }
    }
  }

  // ---- offsets: off(n,g) * sum of the group's activations
  if (d.offset_mode != 0) {
    for (int g = g0; g < g1; ++g) {
      float xs[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float v = 0.f;
        for (int pi = lane; pi < G / 2; pi += kWave) v = dot2(xr[m][g * (G / 2) + pi], 0x3C003C00u, v);
        xs[m] = wave_sum(v);
      }
      if (row_ok) {
        const float o = h2f(d.offset_mode == 1 ? d.offset[row] : d.offset[(size_t)row * d.ng + g]);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = fmaf(o, xs[m], acc[m]);
      }
    }
  }

  if (!row_ok) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < d.m) {
      if (d.splits > 1) {
        d.partial[((size_t)split * d.m + m) * d.n + row] = acc[m];
      } else if (d.y_f32) {
        reinterpret_cast<float*>(d.y)[(size_t)m * d.n + row] = acc[m];
      } else {
        reinterpret_cast<_Float16*>(d.y)[(size_t)m * d.n + row] = (_Float16)acc[m];
      }
    }
  }
}

__global__ void splitk_reduce_kernel(const float* __restrict__ partial, int splits, int m, int n,
                                     void* y, int y_f32) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)m * n;
  if (i >= total) return;
  float s = 0.f;
  for (int p = 0; p < splits; ++p) s += partial[(size_t)p * total + i];
  if (y_f32)
    reinterpret_cast<float*>(y)[i] = s;
  else
    reinterpret_cast<_Float16*>(y)[i] = (_Float16)s;
}

template <int FMT, int G>
hipError_t launch_fmt_g(int mt, const GemvDesc* descs, int ndesc, const GemvDesc& one, int items,
                        hipStream_t s) {
  const size_t lds = (size_t)kGemvRows * Geo<FMT, G>::PITCH;
  switch (mt) {
    case 1: hipLaunchKernelGGL((gemv_kernel<FMT, G, 1>), dim3(items), dim3(kWave), lds, s, descs, ndesc, one); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<FMT, G, 2>), dim3(items), dim3(kWave), lds, s, descs, ndesc, one); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<FMT, G, 4>), dim3(items), dim3(kWave), lds, s, descs, ndesc, one); break;
    case 8: hipLaunchKernelGGL((gemv_kernel<FMT, G, 8>), dim3(items), dim3(kWave), lds, s, descs, ndesc, one); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int gemv_stage_bytes(int format, int group) {
  // groups per stage; split boundaries must be multiples of this
  if (format == 0) return group == 64 ? Geo<0, 64>::SG : Geo<0, 128>::SG;
  return group == 64 ? Geo<1, 64>::SG : Geo<1, 128>::SG;
}

hipError_t launch_gemv(int format, int group, int mt, const GemvDesc* descs, int ndesc,
                       const GemvDesc& one, int total_items, int /*max_stage_bytes*/,
                       hipStream_t s) {
  if (total_items <= 0) return hipSuccess;
  if (format == 0 && group == 64) return launch_fmt_g<0, 64>(mt, descs, ndesc, one, total_items, s);
  if (format == 0 && group == 128) return launch_fmt_g<0, 128>(mt, descs, ndesc, one, total_items, s);
  if (format == 1 && group == 64) return launch_fmt_g<1, 64>(mt, descs, ndesc, one, total_items, s);
  if (format == 1 && group == 128) return launch_fmt_g<1, 128>(mt, descs, ndesc, one, total_items, s);
  return hipErrorInvalidValue;
}

hipError_t launch_splitk_reduce(const float* partial, int splits, int m, int n, void* y, int y_f32,
                                hipStream_t s) {
  const size_t total = (size_t)m * n;
  if (!total) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     partial, splits, m, n, y, y_f32);
  return hipGetLastError();
}

}  // namespace tern
