// Base-3 decode product y = x W^T for up to 4 activation rows, with the
// multiply-adds on the matrix cores (direct ternary execution: "Can ternary
// LLMs hit 1.58 bits per weight", How It Works; arXiv 2609.09240, packed
// weights consumed directly).
//
// Work split.  A workgroup of 8 wavefronts stays on its CU for the whole
// launch (one per CU: the table and stage buffers below take most of the
// LDS).  Each wavefront walks its own list of work items; an item is 64
// output rows (one per lane) times a range of 208-byte stages of their packed
// rows (8 groups of 128 trits, or 16 of 64).
//
// Stream.  A stage of the wavefront's 64 rows goes from HBM straight into
// its LDS buffer with 16-byte LDS-direct buffer loads (no registers); each
// lane then reads its own row's 208 bytes from LDS (row pitch 208 bytes:
// conflict-free 16-byte reads) and the next stage is requested right away,
// so one stage per wavefront is always in flight while one is computed.
//
// Decode.  A base-3 byte holds five trits.  One 16-byte LDS table entry per
// byte value holds them as FP16: (t0, t1), (t2, t3), (t4, 0), (0, t4).  The
// table is stored kLutCopies times, lane l reading copy l % kLutCopies, so
// that the random byte values of a wavefront spread over the LDS banks.
//
// Products.  v_mfma_f32_4x4x4_16b_f16 with the A operand broadcast from one
// block (cbsz = 4): the 16 blocks of 4 lanes each take 4 trits of their 4
// output rows, so every lane multiplies its own row, and the broadcast block
// supplies 4 activation slots of up to 4 activation rows.  Four bytes feed
// five instructions: t0..t3 of each byte, then the four t4's, assembled by
// two ORs of the (t4, 0) and (0, t4) words.  The activations are prepared
// once per product in the same slot order ("x5" below): per group, per quad
// of bytes j..j+3, chunks (x[5j..5j+3]), ..., (x[5(j+3)..5(j+3)+3]),
// (x[5j+4], x[5j+9], x[5j+14], x[5j+19]); a group's last bytes (26 = 6 quads
// + 2 at group 128) follow the same pattern with zero slots; positions past
// the group are zero.  A register of 16 such chunks serves 16 instructions
// (abid = chunk % 16).
//
// Scales.  Each group's products accumulate in their own registers (two,
// alternating, so consecutive instructions do not wait on each other); at the
// group's end they are scaled by the row's FP16 group scale and added to the
// row's FP32 accumulator.  Residual planes are processed compacted (one lane
// per block, decode_common.h), offsets from FP32 group sums of x prepared
// with x5.  Sums are in a fixed order, so results are bitwise reproducible.
#include <algorithm>
#include <type_traits>

#include "decode_common.h"
#include "internal.h"
#include "kparts.h"

namespace tern {
namespace {

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

constexpr int kB3Threads = kWave * kB3Waves;
constexpr int kStageBytes = 208;                 // bytes per row per stage (lcm of 16 and the 26-byte group)
constexpr int kStageChunks = kStageBytes / 16;   // 16-byte loads per row per stage
constexpr int kStageLds = kGemvRows * kStageBytes;
#ifndef TERN_B3_AUX
#define TERN_B3_AUX 0   // cache policy of the weight stream loads
#endif
#ifndef TERN_B3_LUT_COPIES
#define TERN_B3_LUT_COPIES 8
#endif
constexpr int kLutCopies = TERN_B3_LUT_COPIES;
constexpr int kLutStride = 16 * kLutCopies;
constexpr int kLutBytes = 256 * kLutStride;
constexpr int kB3Lds = kLutBytes + kB3Waves * kStageLds;
static_assert(kB3Lds + 64 <= 160 * 1024, "table and stage buffers must fit the LDS of one CU");

template <int G>
struct B3Geo {
  static constexpr int GB = (G + 4) / 5;                // bytes per group (26, 13)
  static constexpr int SG = kStageBytes / GB;           // groups per stage (8, 16)
  static constexpr int Q = GB / 4;                      // whole quads of bytes per group
  static constexpr int T = GB % 4;                      // bytes after the quads
  // the tail's t4 chunk exists when the first tail byte's t4 lies inside the group
  static constexpr int T4 = (T > 0 && 5 * 4 * Q + 4 < G) ? 1 : 0;
  static constexpr int CPG = 5 * Q + T + T4;            // chunks (instructions) per group (33, 16)
  static constexpr int CPS = CPG * SG;                  // chunks per stage
  static constexpr int AREG = (CPS + 15) / 16;          // A registers per stage
  static constexpr int SCW = SG / 8;                    // 16-byte scale loads per stage
  static_assert(SG * GB == kStageBytes, "a stage holds whole groups");
};

__device__ __forceinline__ h4_t as_h4(u2_t v) { return __builtin_bit_cast(h4_t, v); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, size_t bytes) {
  const uint32_t n = (uint32_t)std::min(bytes, (size_t)0xFFFFFFF0u);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

// Table entry of byte value v: (t0, t1), (t2, t3), (t4, 0), (0, t4) as FP16
// pairs, with t_i = digit i (least significant first) minus one; values above
// 242 are not encodings and map to zero.
__device__ u4_t b3_lut_entry(int v) {
  if (v >= 243) return u4_t{0u, 0u, 0u, 0u};
  uint32_t h[5];
  for (int i = 0; i < 5; ++i) {
    const int dg = v % 3;
    v /= 3;
    h[i] = dg == 0 ? 0xBC00u : dg == 2 ? 0x3C00u : 0u;
  }
  return u4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4], h[4] << 16};
}

// Position within its group of slot h of chunk c, or -1 for a zero slot.
template <int G>
__device__ __forceinline__ int x5_pos(int c, int h) {
  using Gm = B3Geo<G>;
  int pos;
  if (c < 5 * Gm::Q) {
    const int q = c / 5, r = c % 5;
    pos = r < 4 ? 5 * (4 * q + r) + h : 5 * (4 * q + h) + 4;
  } else {
    const int t = c - 5 * Gm::Q;
    if (t < Gm::T) pos = 5 * (4 * Gm::Q + t) + h;
    else pos = h < Gm::T ? 5 * (4 * Gm::Q + h) + 4 : -1;
  }
  return pos >= 0 && pos < G ? pos : -1;
}

// One block per (product, activation row): x5 chunks of the row and, when
// asked for, the FP32 sums of every group (in position order).
template <int G>
__global__ __launch_bounds__(256) void b3_prep_kernel(const B3Prep* __restrict__ preps, B3Prep one) {
  using Gm = B3Geo<G>;
  const B3Prep p = preps ? preps[blockIdx.x / 4] : one;
  const int m = blockIdx.x % 4;
  if (m >= p.m) return;
  const int ng = p.k / G;
  const uint16_t* xr = p.x + (size_t)m * p.k;
  uint16_t* o = p.x5 + (size_t)m * ng * Gm::CPG * 4;
  for (int c = threadIdx.x; c < ng * Gm::CPG; c += 256) {
    const int g = c / Gm::CPG, cc = c % Gm::CPG;
    uint32_t v[2];
    for (int hp = 0; hp < 2; ++hp) {
      const int p0 = x5_pos<G>(cc, 2 * hp), p1 = x5_pos<G>(cc, 2 * hp + 1);
      const uint32_t a = p0 >= 0 ? xr[g * G + p0] : 0u, b = p1 >= 0 ? xr[g * G + p1] : 0u;
      v[hp] = a | (b << 16);
    }
    *reinterpret_cast<u2_t*>(o + (size_t)c * 4) = u2_t{v[0], v[1]};
  }
  if (p.xs) {
    for (int g = threadIdx.x; g < ng; g += 256) {
      float s = 0.f;
      for (int i = 0; i < G; ++i) s += h2f(xr[g * G + i]);
      p.xs[(size_t)m * ng + g] = s;
    }
  }
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes dst + 16 l
// (dst the same in every lane); counted by vmcnt like a load.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, TERN_B3_AUX);
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }      // vmcnt(0)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }    // lgkmcnt(0)

// The table entry of byte o (0..207) of this lane's stage row W.
__device__ __forceinline__ u4_t lut_at(const uint8_t* lut_lane, const uint32_t (&W)[kStageBytes / 4], int o) {
  const uint32_t v = (W[o >> 2] >> (8 * (o & 3))) & 0xFFu;
  return *reinterpret_cast<const u4_t*>(lut_lane + v * kLutStride);
}

template <int G>
struct StageRegs {
  u2_t a[B3Geo<G>::AREG];   // activation chunks (A operands)
  u4_t sc[B3Geo<G>::SCW];   // FP16 group scales of the lane's row
};

// Compile-time loop: f(integral_constant<int, I>) for I in [I0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor<I + 1, N>(f);
  }
}

// Instruction for chunk T of the stage: A register T / 16, broadcast block T % 16.
template <int T>
__device__ __forceinline__ f4_t mfma_chunk(const u2_t* a, u2_t b, f4_t acc) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(a[T >> 4]), as_h4(b), acc, 4, T & 15, 0);
}

// Group Gi of the stage: its 26 (13) bytes through the table and the matrix
// cores, then the row's group scale onto the FP32 accumulators.
template <int G, int MT, int Gi>
__device__ __forceinline__ void b3_group(const uint8_t* lut_lane, const uint32_t (&W)[kStageBytes / 4],
                                         const StageRegs<G>& R, float (&acc)[MT]) {
  using Gm = B3Geo<G>;
  constexpr int o0 = Gi * Gm::GB;    // first byte of the group in the stage
  constexpr int t0 = Gi * Gm::CPG;   // first chunk of the group in the stage
  f4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
  sfor<0, Gm::Q>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    u4_t e[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) e[b] = lut_at(lut_lane, W, o0 + 4 * q + b);
    D0 = mfma_chunk<t0 + 5 * q + 0>(R.a, u2_t{e[0].x, e[0].y}, D0);
    D1 = mfma_chunk<t0 + 5 * q + 1>(R.a, u2_t{e[1].x, e[1].y}, D1);
    D0 = mfma_chunk<t0 + 5 * q + 2>(R.a, u2_t{e[2].x, e[2].y}, D0);
    D1 = mfma_chunk<t0 + 5 * q + 3>(R.a, u2_t{e[3].x, e[3].y}, D1);
    D0 = mfma_chunk<t0 + 5 * q + 4>(R.a, u2_t{e[0].z | e[1].w, e[2].z | e[3].w}, D0);
  });
  if constexpr (Gm::T > 0) {
    constexpr int tt = t0 + 5 * Gm::Q;
    const u4_t e0 = lut_at(lut_lane, W, o0 + 4 * Gm::Q);
    D1 = mfma_chunk<tt>(R.a, u2_t{e0.x, e0.y}, D1);
    if constexpr (Gm::T == 2) {
      const u4_t e1 = lut_at(lut_lane, W, o0 + 4 * Gm::Q + 1);
      D0 = mfma_chunk<tt + 1>(R.a, u2_t{e1.x, e1.y}, D0);
      if constexpr (Gm::T4) D1 = mfma_chunk<tt + 2>(R.a, u2_t{e0.z | e1.w, 0u}, D1);
    } else {
      static_assert(Gm::T == 1 || Gm::T == 2, "tails of one or two bytes");
      if constexpr (Gm::T4) D0 = mfma_chunk<tt + 1>(R.a, u2_t{e0.z, 0u}, D0);
    }
  }
  const uint32_t sw = R.sc[Gi / 8][(Gi % 8) / 2];
  const float s = h2f((uint16_t)(Gi % 2 ? sw >> 16 : sw & 0xFFFFu));
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = fmaf(s, D0[i] + D1[i], acc[i]);
}

template <int G, int MT>
__global__ __launch_bounds__(kB3Threads) void gemv_b3_kernel(const GemvDesc* __restrict__ descs,
                                                             const B3Item* __restrict__ items,
                                                             const uint32_t* __restrict__ wbeg, GemvDesc one,
                                                             int one_items) {
  using Gm = B3Geo<G>;
  __shared__ uint4 b3_smem[kB3Lds / 16];
  uint8_t* lds = reinterpret_cast<uint8_t*>(b3_smem);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;

  for (int e = tid; e < 256 * kLutCopies; e += kB3Threads)
    *reinterpret_cast<u4_t*>(lds + (e / kLutCopies) * kLutStride + (e % kLutCopies) * 16) = b3_lut_entry(e / kLutCopies);
  __syncthreads();

  uint8_t* buf = lds + kLutBytes + wave * kStageLds;
  const uint8_t* lut_lane = lds + (lane % kLutCopies) * 16;
  const int gw = (int)blockIdx.x * kB3Waves + wave;
  int it = gw, it_end = one_items, it_step = (int)gridDim.x * kB3Waves;
  if (descs) {
    it = (int)wbeg[gw];
    it_end = (int)wbeg[gw + 1];
    it_step = 1;
  }

  for (; it < it_end; it += it_step) {
    GemvDesc d;
    int rb, part;
    if (descs) {
      const B3Item e = items[it];
      d = descs[e.dp >> 16];
      part = (int)(e.dp & 0xFFFFu);
      rb = (int)e.rb;
    } else {
      d = one;
      rb = it % d.row_blocks;
      part = it / d.row_blocks;
    }
    const int row0 = rb * kGemvRows;
    const int row = row0 + lane;
    const bool row_ok = row < d.n;
    const int nst = (d.ng + Gm::SG - 1) / Gm::SG;
    const int s0 = part * d.gps, s1 = min(nst, s0 + d.gps);
    const int ga = s0 * Gm::SG, gb = min(d.ng, s1 * Gm::SG);

    const __amdgpu_buffer_rsrc_t rw = rsrc(d.plane0 + (size_t)row0 * d.stride, (size_t)(d.n - row0) * d.stride);
    const __amdgpu_buffer_rsrc_t rs = rsrc(d.scale0 + (size_t)row0 * d.ng, (size_t)(d.n - row0) * d.ng * 2);
    const size_t x5row = (size_t)d.ng * Gm::CPG * 8;   // bytes per activation row of x5
    const __amdgpu_buffer_rsrc_t rx = rsrc(d.x5, x5row * d.m);
    // the lane's share of a stage's loads: chunk 64 u + lane = (row, 16-byte column)
    uint32_t voff[kStageChunks];
#pragma unroll
    for (int u = 0; u < kStageChunks; ++u) {
      const int c = 64 * u + lane;
      voff[u] = (uint32_t)(c / kStageChunks) * (uint32_t)d.stride + (uint32_t)(c % kStageChunks) * 16u;
    }
    const uint32_t svoff = (uint32_t)lane * (uint32_t)d.ng * 2u;
    const uint32_t avoff = (uint32_t)min(lane % 4, d.m - 1) * (uint32_t)x5row + (uint32_t)(lane / 4) * 8u;

    auto issue = [&](int s, StageRegs<G>& R) {
#pragma unroll
      for (int u = 0; u < kStageChunks; ++u) lds_load16(rw, buf + 1024 * u, voff[u] + (uint32_t)s * kStageBytes);
      // scales: 16-byte loads when every row's scales start on a dword (an
      // unaligned dword that straddles the end of the array would read as
      // zero); one load per scale otherwise
      if ((d.ng & 1) == 0) {
#pragma unroll
        for (int w = 0; w < Gm::SCW; ++w)
          R.sc[w] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, svoff + (uint32_t)(s * Gm::SG) * 2u + 16u * w, 0, 0));
      } else {
#pragma unroll
        for (int w = 0; w < Gm::SCW; ++w) {
          uint32_t h[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            h[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, svoff + (uint32_t)(s * Gm::SG + 8 * w + j) * 2u, 0, 0);
          R.sc[w] = u4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
      }
#pragma unroll
      for (int u = 0; u < Gm::AREG; ++u)
        R.a[u] = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(rx, avoff + (uint32_t)(s * Gm::CPS) * 8u + 128u * u, 0, 0));
    };

    float acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = 0.f;

    auto body = [&](int s, StageRegs<G>& Rc, StageRegs<G>& Rn) {
      wait_vm0();    // stage s is in LDS; its scales and activations are in Rc
      wave_sync();
      uint32_t W[kStageBytes / 4];
#pragma unroll
      for (int q = 0; q < kStageChunks; ++q) {
        const u4_t v = *reinterpret_cast<const u4_t*>(buf + lane * kStageBytes + 16 * q);
        W[4 * q] = v.x; W[4 * q + 1] = v.y; W[4 * q + 2] = v.z; W[4 * q + 3] = v.w;
      }
      wait_lgkm0();  // the buffer is free for the next stage
      wave_sync();
      if (s + 1 < s1) issue(s + 1, Rn);
      const int gs = s * Gm::SG;
      sfor<0, Gm::SG>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        if (gs + g < gb) b3_group<G, MT, g>(lut_lane, W, Rc, acc);
      });
    };

    if (s0 < s1) {
      StageRegs<G> RA, RB;
      wait_lgkm0();
      wave_sync();
      issue(s0, RA);
      int s = s0;
      for (; s + 1 < s1; s += 2) {
        body(s, RA, RB);
        body(s + 1, RB, RA);
      }
      if (s < s1) body(s, RA, RB);
    }

    // ---- residual planes and offsets over the item's groups [ga, gb)
    const GLOBAL uint32_t* xr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xr[m] = reinterpret_cast<const GLOBAL uint32_t*>(gp(d.x) + (size_t)min(m, d.m - 1) * d.k);
    if (gb > ga) {
      if (d.planes > 1) residual_compact<G, MT>(d, 0, row, row_ok, ga, gb, xr, buf, kStageLds, acc);
      if (d.planes > 2) residual_compact<G, MT>(d, 1, row, row_ok, ga, gb, xr, buf, kStageLds, acc);
      if (d.offset_mode != 0 && row_ok) {
        const GLOBAL uint16_t* off = gp(d.offset);
        const GLOBAL float* xs = gp(d.xs);
        if (d.offset_mode == 1) {
          const float o = h2f(off[row]);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            float sx = 0.f;
            for (int g = ga; g < gb; ++g) sx += xs[(size_t)min(m, d.m - 1) * d.ng + g];
            acc[m] = fmaf(o, sx, acc[m]);
          }
        } else {
          for (int g = ga; g < gb; ++g) {
            const float o = h2f(off[(size_t)row * d.ng + g]);
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = fmaf(o, xs[(size_t)min(m, d.m - 1) * d.ng + g], acc[m]);
          }
        }
      }
    }
    wave_sync();

    // ---- output, or this part's partial sums (summed by the row block's last part)
    if (d.splits > 1) {
      if (row_ok) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < d.m) part_store(d.partial + ((size_t)part * d.m + m) * d.n + row, acc[m]);
      }
      if (d.ctr == nullptr || !last_part_wave(d.ctr + rb, d.splits, lane)) continue;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < d.m && row_ok) {
          float v = 0.f;
          for (int sp = 0; sp < d.splits; ++sp) v += part_load(d.partial + ((size_t)sp * d.m + m) * d.n + row);
          acc[m] = v;
        }
      }
    }
    if (row_ok) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < d.m) {
          if (d.y_f32) reinterpret_cast<float*>(d.y)[(size_t)m * d.n + row] = acc[m];
          else reinterpret_cast<_Float16*>(d.y)[(size_t)m * d.n + row] = (_Float16)acc[m];
        }
      }
    }
  }
}

template <int G, int MT>
hipError_t launch_b3_mt(const GemvDesc* descs, const B3Item* items, const uint32_t* wbeg, int nwg, const GemvDesc& one,
                        int one_items, hipStream_t s) {
  hipLaunchKernelGGL((gemv_b3_kernel<G, MT>), dim3(nwg), dim3(kB3Threads), 0, s, descs, items, wbeg, one,
                     one_items);
  return hipGetLastError();
}

template <int G>
hipError_t launch_b3_g(int mt, const GemvDesc* descs, const B3Item* items, const uint32_t* wbeg, int nwg,
                       const GemvDesc& one, int one_items, hipStream_t s) {
  switch (mt) {
    case 1: return launch_b3_mt<G, 1>(descs, items, wbeg, nwg, one, one_items, s);
    case 2: return launch_b3_mt<G, 2>(descs, items, wbeg, nwg, one, one_items, s);
    case 4: return launch_b3_mt<G, 4>(descs, items, wbeg, nwg, one, one_items, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int b3_chunks_per_group(int group) { return group == 64 ? B3Geo<64>::CPG : B3Geo<128>::CPG; }
int b3_stage_groups(int group) { return group == 64 ? B3Geo<64>::SG : B3Geo<128>::SG; }

hipError_t launch_b3_prep(int group, const B3Prep* preps, int count, const B3Prep& one, hipStream_t s) {
  const int blocks = (preps ? count : 1) * 4;
  if (blocks <= 0) return hipSuccess;
  if (group == 64) hipLaunchKernelGGL(b3_prep_kernel<64>, dim3(blocks), dim3(256), 0, s, preps, one);
  else if (group == 128) hipLaunchKernelGGL(b3_prep_kernel<128>, dim3(blocks), dim3(256), 0, s, preps, one);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemv_b3(int group, int mt, const GemvDesc* descs, const B3Item* items, const uint32_t* wbeg, int nwg,
                          const GemvDesc& one, int one_items, hipStream_t s) {
  if (nwg <= 0) return hipSuccess;
  if (group == 64) return launch_b3_g<64>(mt, descs, items, wbeg, nwg, one, one_items, s);
  if (group == 128) return launch_b3_g<128>(mt, descs, items, wbeg, nwg, one, one_items, s);
  return hipErrorInvalidValue;
}

}  // namespace tern
