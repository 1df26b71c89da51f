// Decode-path product y = x W^T for a few activation rows (M <= 8 per pass)
// on packed ternary planes: the direct ternary product ("Can ternary LLMs hit
// 1.58 bits per weight", How It Works: matrix products become additions and
// subtractions; arXiv 2609.09240: the packed weights are consumed directly).
//
// One row per lane: a wavefront covers 64 output rows.  Packed rows are staged through LDS with coalesced 16-byte
// loads (8 or 13 lanes cover 128 or 208 contiguous bytes of a row), then each
// lane decodes its own row.  All lanes sit at the same K position, so the
// activations are wave-uniform and are read with scalar loads into SGPRs,
// which leaves the VALU for decode and multiply-accumulate only.
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
//
// Work item = 64 rows x one K split, run by a workgroup of 4 wavefronts that
// split the item's groups between them; their FP32 accumulators are summed
// in wave order through LDS (deterministic, no global memory fences: on this
// multi-XCD part a device-scope fence writes back and invalidates the L2).
// When a row block is additionally split along K across workgroups, each
// split writes FP32 partials and a second kernel sums them in split order.
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

template <int FMT, int G>
struct Geo {
  static constexpr int GB = FMT == 0 ? G / 4 : (G + 4) / 5;   // bytes per group
  static constexpr int SGB = FMT == 0 ? 128 : 208;             // bytes per row per stage
  static constexpr int SG = SGB / GB;                           // groups per stage
  static constexpr int CPR = SGB / 16;                          // 16-byte chunks per row
  static constexpr int PITCH = FMT == 0 ? 144 : 208;            // LDS row pitch (bytes)
  static constexpr int CHUNKS = kGemvRows * CPR / kWave;        // chunks per lane per stage
  static constexpr int XDW = SG * G / 2;                        // activation dwords per stage per row of x
  static constexpr int XCH = XDW / 4 / kWave;                   // 16-byte x chunks per lane per stage
  static constexpr int WBYTES = kGemvRows * PITCH;              // weight part of the LDS stage
  static_assert(SG * GB == SGB, "stage must hold whole groups");
  static_assert((PITCH / 16) % 2 == 1, "odd 16-byte pitch keeps b128 reads conflict-free");
};

// Base-3 byte -> 2-bit codes.  For a byte pair (A, B) holding trits t0..t4 and
// t5..t9, pair i = (t[2i], t[2i+1]) must sit at bits 6+2i (low) and 22+2i
// (high) of lutA[A] | lutB[B]; then pair i decodes with shift 8-2i.
__device__ void build_b3_entry(int v, uint32_t* lutA, uint32_t* lutB) {
  {
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

__device__ __forceinline__ int find_desc(const GemvDesc* __restrict__ descs, int ndesc, int item) {
  int lo = 0, hi = ndesc - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (descs[mid].tile_begin <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Residual blocks of this lane's row in groups [g0, g1) of plane p.
template <int G, int MT>
__device__ __forceinline__ void residual_plane(const GemvDesc& d, int p, int row, int g0, int g1,
                                               const GLOBAL uint32_t* const (&xr)[MT],
                                               float (&acc)[MT]) {
  const GLOBAL uint32_t* rm = gp(d.mask[p]) + (size_t)row * d.mwords;
  uint32_t b = gp(d.rowptr[p])[row];
  for (int w = 0; w < (g0 >> 5); ++w) b += __popc(rm[w]);
  if (g0 & 31) b += __popc(rm[g0 >> 5] & ((1u << (g0 & 31)) - 1u));
  const GLOBAL uint8_t* blocks = gp(d.blocks[p]);
  const GLOBAL uint16_t* rscale = gp(d.rscale[p]);
  for (int w = g0 >> 5; w <= ((g1 - 1) >> 5); ++w) {
    uint32_t bits = rm[w];
    const int lo = max(g0 - (w << 5), 0), hi = min(g1 - (w << 5), 32);
    bits &= (lo > 0 ? ~((1u << lo) - 1u) : ~0u) & (hi < 32 ? ((1u << hi) - 1u) : ~0u);
    while (bits) {
      const int g = (w << 5) + __builtin_ctz(bits);
      bits &= bits - 1u;
      const GLOBAL u4_t* blk = reinterpret_cast<const GLOBAL u4_t*>(blocks + (size_t)b * (G / 4));
      float part[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) part[m] = 0.f;
#pragma unroll
      for (int q = 0; q < G / 64; ++q) {
        const u4_t v = blk[q];
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
      for (int m = 0; m < MT; ++m) acc[m] = fmaf(rs, part[m], acc[m]);
      ++b;
    }
  }
}

constexpr int kWaves = 4;  // wavefronts per workgroup, splitting K

__device__ __forceinline__ void wave_sync() {
  // LDS traffic of one wavefront is processed in order; this keeps the
  // compiler from moving LDS accesses across the hand-off point.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int FMT, int G, int MT>
__global__ __launch_bounds__(kWave * kWaves) void gemv_kernel(const GemvDesc* __restrict__ descs,
                                                              int ndesc, GemvDesc one) {
  using Gm = Geo<FMT, G>;
  extern __shared__ uint4 stage_all[];  // per wave: [64 rows][PITCH] + activations of a stage
  __shared__ uint32_t lutA[FMT == 1 ? 256 : 1];
  __shared__ uint32_t lutB[FMT == 1 ? 256 : 1];

  const int item_g = blockIdx.x;
  GemvDesc d;
  if (ndesc > 0) d = descs[find_desc(descs, ndesc, item_g)];
  else d = one;
  const int item = item_g - d.tile_begin;
  const int rb = item % d.row_blocks;
  const int split = item / d.row_blocks;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int row = rb * kGemvRows + lane;
  const bool row_ok = row < d.n;
  // this wave's share of the item's groups, on stage boundaries
  const int ga = split * d.gps;
  const int gb = min(d.ng, ga + d.gps);
  const int q = ((gb - ga + kWaves - 1) / kWaves + Gm::SG - 1) / Gm::SG * Gm::SG;
  const int g0 = min(gb, ga + wave * q);
  const int g1 = min(gb, g0 + q);
  const int nstages = (g1 - g0 + Gm::SG - 1) / Gm::SG;

  if (FMT == 1) {
    for (int v = threadIdx.x; v < 256; v += kWave * kWaves) build_b3_entry(v, lutA, lutB);
    __syncthreads();
  }

  const GLOBAL uint32_t* xr[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
    xr[m] = reinterpret_cast<const GLOBAL uint32_t*>(gp(d.x) + (size_t)min(m, d.m - 1) * d.k);

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;

  const GLOBAL uint8_t* prow0 = gp(d.plane0) + (size_t)rb * kGemvRows * d.stride;
  const GLOBAL uint16_t* srow = gp(d.scale0) + (size_t)(row_ok ? row : 0) * d.ng;
  const int rows_here = min(kGemvRows, d.n - rb * kGemvRows);
  uint8_t* lds = reinterpret_cast<uint8_t*>(stage_all) + (size_t)wave * (Gm::WBYTES + MT * Gm::XDW * 4);

  // prefetch registers for the next stage: packed rows, scales, activations
  u4_t pre[Gm::CHUNKS];
  uint16_t spre[Gm::SG];
  u4_t xpre[MT][Gm::XCH];
  const GLOBAL u4_t* xq[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xq[m] = reinterpret_cast<const GLOBAL u4_t*>(xr[m]);
#define TERN_LOAD_STAGE(s_)                                                                 \
  do {                                                                                      \
    const int gs_ = g0 + (s_) * Gm::SG;                                                     \
    const int bytes_ = min(Gm::SG, g1 - gs_) * Gm::GB;                                      \
    const GLOBAL uint8_t* base_ = prow0 + (size_t)gs_ * Gm::GB;                             \
    _Pragma("unroll") for (int i = 0; i < Gm::CHUNKS; ++i) {                                \
      const int c = i * kWave + lane;                                                       \
      const int r = c / Gm::CPR, col = c % Gm::CPR;                                         \
      if (r < rows_here && col * 16 < bytes_)                                               \
        pre[i] = *reinterpret_cast<const GLOBAL u4_t*>(base_ + (size_t)r * d.stride + col * 16); \
    }                                                                                       \
    _Pragma("unroll") for (int j = 0; j < Gm::SG; ++j)                                      \
      spre[j] = (row_ok && gs_ + j < g1) ? srow[gs_ + j] : (uint16_t)0;                     \
    _Pragma("unroll") for (int m = 0; m < MT; ++m)                                          \
      _Pragma("unroll") for (int i = 0; i < Gm::XCH; ++i) {                                 \
        const int xc_ = gs_ * (G / 8) + i * kWave + lane;                                   \
        if (xc_ < g1 * (G / 8)) xpre[m][i] = xq[m][xc_];                                    \
      }                                                                                     \
  } while (0)

  if (nstages > 0) TERN_LOAD_STAGE(0);
  for (int s = 0; s < nstages; ++s) {
    const int gs = g0 + s * Gm::SG;
    const int ngs = min(Gm::SG, g1 - gs);
    wave_sync();  // previous stage consumed
#pragma unroll
    for (int i = 0; i < Gm::CHUNKS; ++i) {
      const int c = i * kWave + lane;
      const int r = c / Gm::CPR, col = c % Gm::CPR;
      *reinterpret_cast<u4_t*>(lds + r * Gm::PITCH + col * 16) = pre[i];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < Gm::XCH; ++i)
        *reinterpret_cast<u4_t*>(lds + Gm::WBYTES + (m * Gm::XDW + (i * kWave + lane) * 4) * 4) = xpre[m][i];
    float sc[Gm::SG];
#pragma unroll
    for (int j = 0; j < Gm::SG; ++j) sc[j] = 0.5f * h2f(spre[j]);
    wave_sync();
    if (s + 1 < nstages) TERN_LOAD_STAGE(s + 1);

    const uint8_t* my = lds + lane * Gm::PITCH;
    // wave-uniform activation chunks of this stage (broadcast LDS reads)
    const u4_t* xs4 = reinterpret_cast<const u4_t*>(lds + Gm::WBYTES);
#pragma unroll
    for (int j = 0; j < Gm::SG; ++j) {
      if (j < ngs) {
        const int g = gs + j;
        float part[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) part[m] = 0.f;
        if (FMT == 0) {
#pragma unroll
          for (int q = 0; q < G / 64; ++q) {
            const u4_t v = *reinterpret_cast<const u4_t*>(my + j * Gm::GB + q * 16);
            const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              u4_t xa[MT], xb[MT];
#pragma unroll
              for (int m = 0; m < MT; ++m) {
                const int c = (m * Gm::XDW + j * (G / 2) + q * 32 + u * 8) / 4;
                xa[m] = xs4[c];
                xb[m] = xs4[c + 1];
              }
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const uint32_t p = pair_of(ws[u], 14 - 2 * i);
#pragma unroll
                for (int m = 0; m < MT; ++m) part[m] = dot2(p, i < 4 ? xa[m][i] : xb[m][i - 4], part[m]);
              }
            }
          }
        } else {
          constexpr int GB = Gm::GB;
          const int off = j * GB;               // compile-time after unrolling
          const int c0 = off >> 4;
          uint32_t dw[12];
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            if (((off + GB - 1) >> 4) >= c0 + q) {
              const u4_t v = *reinterpret_cast<const u4_t*>(my + (c0 + q) * 16);
              dw[4 * q + 0] = v.x; dw[4 * q + 1] = v.y; dw[4 * q + 2] = v.z; dw[4 * q + 3] = v.w;
            } else {
              dw[4 * q + 0] = dw[4 * q + 1] = dw[4 * q + 2] = dw[4 * q + 3] = 0u;
            }
          }
          const int sh = off - c0 * 16;
          u4_t xc[MT][5];
#pragma unroll
          for (int bp = 0; bp < (GB + 1) / 2; ++bp) {
            if (bp % 4 == 0) {  // activation pairs 5*bp .. 5*bp+19 of the group
#pragma unroll
              for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int c = 0; c < 5; ++c)
                  if (4 * (5 * bp / 4 + c) < G / 2) xc[m][c] = xs4[(m * Gm::XDW + j * (G / 2)) / 4 + 5 * bp / 4 + c];
            }
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
                const int xi = 5 * bp + i - 4 * (5 * (bp / 4 * 4) / 4);  // index within the 5 chunks
#pragma unroll
                for (int m = 0; m < MT; ++m) part[m] = dot2(p, xc[m][xi / 4][xi % 4], part[m]);
              }
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = fmaf(sc[j], part[m], acc[m]);
      }
    }
  }
#undef TERN_LOAD_STAGE

  // ---- residual planes: each lane walks its row's compact blocks in [g0, g1)
  if (row_ok && g1 > g0) {
    if (d.planes > 1) residual_plane<G, MT>(d, 0, row, g0, g1, xr, acc);
    if (d.planes > 2) residual_plane<G, MT>(d, 1, row, g0, g1, xr, acc);
  }

  // ---- offsets: off(n,g) * sum of the group's activations
  if (d.offset_mode != 0) {
    const GLOBAL uint16_t* off = gp(d.offset);
    for (int g = g0; g < g1; ++g) {
      float xs[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float v = 0.f;
        for (int pi = lane; pi < G / 2; pi += kWave) v = dot2(xr[m][g * (G / 2) + pi], 0x3C003C00u, v);
        xs[m] = wave_sum(v);
      }
      if (row_ok) {
        const float o = h2f(d.offset_mode == 1 ? off[row] : off[(size_t)row * d.ng + g]);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = fmaf(o, xs[m], acc[m]);
      }
    }
  }

  // ---- combine the wavefronts' accumulators in wave order
  __syncthreads();  // every wave is done with its stage buffers
  float* red = reinterpret_cast<float*>(stage_all);
#pragma unroll
  for (int m = 0; m < MT; ++m) red[(wave * MT + m) * kWave + lane] = acc[m];
  __syncthreads();
  if (wave != 0 || !row_ok) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float v = red[m * kWave + lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += red[(w * MT + m) * kWave + lane];
    acc[m] = v;
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < d.m) {
      if (d.splits > 1)
        d.partial[((size_t)split * d.m + m) * d.n + row] = acc[m];
      else if (d.y_f32)
        reinterpret_cast<float*>(d.y)[(size_t)m * d.n + row] = acc[m];
      else
        reinterpret_cast<_Float16*>(d.y)[(size_t)m * d.n + row] = (_Float16)acc[m];
    }
  }
}

__global__ void splitk_reduce_kernel(const float* __restrict__ partial, int splits, int m, int n,
                                     void* y, int y_f32) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)m * n;
  if (i >= total) return;
  float v = 0.f;
  for (int s = 0; s < splits; ++s) v += partial[(size_t)s * total + i];
  if (y_f32) reinterpret_cast<float*>(y)[i] = v;
  else reinterpret_cast<_Float16*>(y)[i] = (_Float16)v;
}

template <int FMT, int G>
hipError_t launch_fmt_g(int mt, const GemvDesc* descs, int ndesc, const GemvDesc& one, int items,
                        hipStream_t s) {
  const size_t lds = (size_t)kWaves * (Geo<FMT, G>::WBYTES + (size_t)mt * Geo<FMT, G>::XDW * 4);
  const dim3 block(kWave * kWaves);
  switch (mt) {
    case 1: hipLaunchKernelGGL((gemv_kernel<FMT, G, 1>), dim3(items), block, lds, s, descs, ndesc, one); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<FMT, G, 2>), dim3(items), block, lds, s, descs, ndesc, one); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<FMT, G, 4>), dim3(items), block, lds, s, descs, ndesc, one); break;
    case 8: hipLaunchKernelGGL((gemv_kernel<FMT, G, 8>), dim3(items), block, lds, s, descs, ndesc, one); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int gemv_stage_groups(int format, int group) {
  // groups per stage; split boundaries must be multiples of this
  if (format == 0) return group == 64 ? Geo<0, 64>::SG : Geo<0, 128>::SG;
  return group == 64 ? Geo<1, 64>::SG : Geo<1, 128>::SG;
}

hipError_t launch_splitk_reduce(const float* partial, int splits, int m, int n, void* y, int y_f32,
                                hipStream_t s) {
  const size_t total = (size_t)m * n;
  if (!total) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     partial, splits, m, n, y, y_f32);
  return hipGetLastError();
}

hipError_t launch_gemv(int format, int group, int mt, const GemvDesc* descs, int ndesc,
                       const GemvDesc& one, int total_items, hipStream_t s) {
  if (total_items <= 0) return hipSuccess;
  if (format == 0 && group == 64) return launch_fmt_g<0, 64>(mt, descs, ndesc, one, total_items, s);
  if (format == 0 && group == 128) return launch_fmt_g<0, 128>(mt, descs, ndesc, one, total_items, s);
  if (format == 1 && group == 64) return launch_fmt_g<1, 64>(mt, descs, ndesc, one, total_items, s);
  if (format == 1 && group == 128) return launch_fmt_g<1, 128>(mt, descs, ndesc, one, total_items, s);
  return hipErrorInvalidValue;
}

}  // namespace tern
