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
// 16 copies of each 16-byte entry fill a 256-byte table row: the 16 lanes an
// LDS cycle serves read distinct banks whatever their byte values, and the
// entry address is the byte value in bits 8..15 (one byte permute).
constexpr int kLutCopies = 16;
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

// x5 chunks and, when asked for, FP32 group sums of activation row m of the
// product p: bx = a block of 256 chunks (one per thread; group sums by the
// threads of block 0, one group each, in position order).
template <int G>
__device__ __forceinline__ void b3_prep_rows(const B3Prep& p, int bx, int m) {
  using Gm = B3Geo<G>;
  if (p.zero && bx == 0 && m == 0)
    for (int i = threadIdx.x; i < p.nzero; i += 256) p.zero[i] = 0u;
  if (m >= p.m) return;
  const int ng = p.k / G;
  const uint16_t* xr = p.x + (size_t)m * p.k;
  const int c = bx * 256 + (int)threadIdx.x;
  if (c < ng * Gm::CPG) {
    const int g = c / Gm::CPG, cc = c % Gm::CPG;
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = x5_pos<G>(cc, q);
      h[q] = pos < 0 ? 0u : xr[g * G + pos];
    }
    *reinterpret_cast<u2_t*>(p.x5 + ((size_t)m * ng * Gm::CPG + c) * 4) = u2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  }
  if (p.xs && bx == 0) {
    for (int g = threadIdx.x; g < ng; g += 256) {
      const u4_t* xg = reinterpret_cast<const u4_t*>(xr + (size_t)g * G);
      u4_t w[G / 8];
#pragma unroll
      for (int i = 0; i < G / 8; ++i) w[i] = xg[i];
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < G / 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s += h2f((uint16_t)(w[i][j] & 0xFFFFu));
          s += h2f((uint16_t)(w[i][j] >> 16));
        }
      p.xs[(size_t)m * ng + g] = s;
    }
  }
}

// (each caller passes a struct it has loaded: choosing between a table
// entry and another struct at run time would copy them to scratch memory)
template <int G>
__global__ __launch_bounds__(256) void b3_prep_kernel(const B3Prep* __restrict__ preps, B3Prep one) {
  const int by = (int)blockIdx.y;
  if (preps) {
    const B3Prep p = preps[by / 4];
    b3_prep_rows<G>(p, (int)blockIdx.x, by % 4);
  } else {
    b3_prep_rows<G>(one, (int)blockIdx.x, by % 4);
  }
}

// The preparation of a rotated plan: blockIdx.y = product, blockIdx.x = a
// span of S = max(B, G) positions (whole R blocks and whole groups) for every
// activation row.  With R: the span's R blocks are copied to LDS with
// contiguous 16-byte loads (rows padded by a word, so that threads reading
// consecutive rows use distinct banks), and each value is row i of its block
// times the block of x, v_dot2_f32_f16 over the FP16 pairs in position order
// (FP32), one FP16 rounding; the values go to xr in position order (the
// residual pass reads them) and to x5 in slot order.  Without R the span is
// copied to x5.  The first span of each product also clears its zero list.
template <int G, int B>
__global__ __launch_bounds__(256) void b3_prep_rot_kernel(const B3Prep* __restrict__ preps) {
  using Gm = B3Geo<G>;
  constexpr int S = B > G ? B : G;
  constexpr int P = B / 2 + 1;  // padded R row pitch in LDS (FP16 pairs)
  constexpr int NC = S * (B / 8) / 256;
  static_assert(NC >= 1 && S * (B / 8) % 256 == 0, "R chunks spread over the threads");
  __shared__ uint32_t rs[S * P];
  __shared__ uint32_t xs2[4 * S / 2];  // [row][S/2] FP16 pairs
  __shared__ uint16_t val[4 * S];      // [row][S]
  const B3Prep p = preps[blockIdx.y];
  const int t = threadIdx.x;
  if (p.zero && blockIdx.x == 0)
    for (int i = t; i < p.nzero; i += 256) p.zero[i] = 0u;
  const int p0 = (int)blockIdx.x * S;
  if (p0 >= p.k) return;
  const int m = p.m;
  // positions of the span inside x: all of them for a rotated product (k is
  // a multiple of B and of G); an unrotated one may end inside the span
  const int len = min(S, p.k - p0);
  for (int e = t; e < m * (S / 8); e += 256) {
    const int r = e / (S / 8), j = e % (S / 8);
    if (8 * j >= len) continue;
    const u4_t v = *reinterpret_cast<const u4_t*>(p.x + (size_t)r * p.k + p0 + 8 * j);
    uint32_t* d = xs2 + r * (S / 2) + 4 * j;
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
  }
  if (p.R) {
    // the span's rows of R are contiguous: S rows of B / 8 chunks
    const u4_t* rg = reinterpret_cast<const u4_t*>(p.R + (size_t)p0 * B);
    u4_t v[NC];
#pragma unroll
    for (int u = 0; u < NC; ++u) v[u] = rg[t + 256 * u];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = t + 256 * u, row = c / (B / 8), q = c % (B / 8);
      uint32_t* d = rs + row * P + 4 * q;
      d[0] = v[u].x;
      d[1] = v[u].y;
      d[2] = v[u].z;
      d[3] = v[u].w;
    }
  }
  __syncthreads();
  for (int e = t; e < m * S; e += 256) {
    const int r = e / S, i = e % S;
    if (i >= len) continue;
    uint16_t h;
    if (p.R) {
      const uint32_t* ri = rs + i * P;
      const uint32_t* xb = xs2 + r * (S / 2) + (i / B) * (B / 2);
      float acc = 0.f;
#pragma unroll 16
      for (int j = 0; j < B / 2; ++j) acc = dot2(ri[j], xb[j], acc);
      h = __builtin_bit_cast(uint16_t, (_Float16)acc);
      p.xr[(size_t)r * p.k + p0 + i] = h;
    } else {
      h = reinterpret_cast<const uint16_t*>(xs2)[r * S + i];
    }
    val[r * S + i] = h;
  }
  __syncthreads();
  const int ng = p.k / G, g0 = p0 / G;
  constexpr int CS = (S / G) * Gm::CPG;  // chunks of the span per activation row
  for (int e = t; e < m * CS; e += 256) {
    const int r = e / CS, c = e % CS, gl = c / Gm::CPG, cc = c % Gm::CPG;
    if (g0 + gl >= ng) continue;
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = x5_pos<G>(cc, q);
      h[q] = pos < 0 ? 0u : val[r * S + gl * G + pos];
    }
    *reinterpret_cast<u2_t*>(p.x5 + ((size_t)(r * ng + g0 + gl) * Gm::CPG + cc) * 4) =
        u2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  }
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes dst + 16 l
// (dst the same in every lane); counted by vmcnt like a load.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, TERN_B3_AUX);
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }      // vmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm() {  // vmcnt(N), N <= 63
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }    // lgkmcnt(0)

// The table entry of byte o (0..207) of this lane's stage row W; coff is
// the lane's copy offset (16 * (lane % 16)) and the table starts at LDS 0.
__device__ __forceinline__ u4_t lut_at(const uint8_t* lds, uint32_t coff, const uint32_t (&W)[kStageBytes / 4], int o) {
  // address = coff | byte << 8: byte 0 from coff, byte 1 from W's byte o % 4
  const uint32_t a = __builtin_amdgcn_perm(W[o >> 2], coff, 0x0C0C0000u | ((4u + (uint32_t)(o & 3)) << 8));
  return *reinterpret_cast<const u4_t*>(lds + a);
}

// Activation chunks of a stage (A operands) and where the next stage's come
// from: register u holds chunks 16u .. 16u+15 and is refilled with the next
// stage's register u right after its last instruction of this stage.
template <int G>
struct StageRegs {
  u2_t a[B3Geo<G>::AREG];
  __amdgpu_buffer_rsrc_t rx;   // the product's x5
  uint32_t next;               // byte offset of the lane's next-stage register 0
};

template <int G>
__device__ __forceinline__ u2_t load_areg(const StageRegs<G>& R, uint32_t off) {
  return __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(R.rx, off, 0, 0));
}

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
__device__ __forceinline__ void b3_group(const uint8_t* lds, uint32_t coff, const uint32_t (&W)[kStageBytes / 4],
                                         const StageRegs<G>& R, const u4_t (&SC)[B3Geo<G>::SCW], float (&acc)[MT]) {
  using Gm = B3Geo<G>;
  constexpr int o0 = Gi * Gm::GB;    // first byte of the group in the stage
  constexpr int t0 = Gi * Gm::CPG;   // first chunk of the group in the stage
  f4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
  sfor<0, Gm::Q>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    u4_t e[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) e[b] = lut_at(lds, coff, W, o0 + 4 * q + b);
    D0 = mfma_chunk<t0 + 5 * q + 0>(R.a, u2_t{e[0].x, e[0].y}, D0);
    D1 = mfma_chunk<t0 + 5 * q + 1>(R.a, u2_t{e[1].x, e[1].y}, D1);
    D0 = mfma_chunk<t0 + 5 * q + 2>(R.a, u2_t{e[2].x, e[2].y}, D0);
    D1 = mfma_chunk<t0 + 5 * q + 3>(R.a, u2_t{e[3].x, e[3].y}, D1);
    D0 = mfma_chunk<t0 + 5 * q + 4>(R.a, u2_t{e[0].z | e[1].w, e[2].z | e[3].w}, D0);
  });
  if constexpr (Gm::T > 0) {
    constexpr int tt = t0 + 5 * Gm::Q;
    const u4_t e0 = lut_at(lds, coff, W, o0 + 4 * Gm::Q);
    D1 = mfma_chunk<tt>(R.a, u2_t{e0.x, e0.y}, D1);
    if constexpr (Gm::T == 2) {
      const u4_t e1 = lut_at(lds, coff, W, o0 + 4 * Gm::Q + 1);
      D0 = mfma_chunk<tt + 1>(R.a, u2_t{e1.x, e1.y}, D0);
      if constexpr (Gm::T4) D1 = mfma_chunk<tt + 2>(R.a, u2_t{e0.z | e1.w, 0u}, D1);
    } else {
      static_assert(Gm::T == 1 || Gm::T == 2, "tails of one or two bytes");
      if constexpr (Gm::T4) D0 = mfma_chunk<tt + 1>(R.a, u2_t{e0.z, 0u}, D0);
    }
  }
  const uint32_t sw = SC[Gi / 8][(Gi % 8) / 2];
  const float s = h2f((uint16_t)(Gi % 2 ? sw >> 16 : sw & 0xFFFFu));
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = fmaf(s, D0[i] + D1[i], acc[i]);
}

// A whole stage as one software pipeline of steps (a quad of bytes, or a
// group's tail bytes): the table entries of step i + P are requested before
// the instructions of step i, so P steps of LDS latency are in flight.
#ifndef TERN_B3_DEPTH
#define TERN_B3_DEPTH 2
#endif
template <int G>
struct B3Steps {
  using Gm = B3Geo<G>;
  static constexpr int SPG = Gm::Q + (Gm::T > 0 ? 1 : 0);   // steps per group
  static constexpr int NS = Gm::SG * SPG;                     // steps per stage
};

template <int G, int I>
__device__ __forceinline__ void b3_load_step(const uint8_t* lds, uint32_t coff, const uint32_t (&W)[kStageBytes / 4], u4_t (&e)[4]) {
  using Gm = B3Geo<G>;
  constexpr int g = I / B3Steps<G>::SPG, r = I % B3Steps<G>::SPG;
  constexpr int nb = r < Gm::Q ? 4 : Gm::T;
  constexpr int o = g * Gm::GB + 4 * r;
#pragma unroll
  for (int b = 0; b < nb; ++b) e[b] = lut_at(lds, coff, W, o + b);
}

template <int G, int I>
__device__ __forceinline__ void b3_mfma_step(const StageRegs<G>& R, const u4_t (&e)[4], f4_t& D0, f4_t& D1) {
  using Gm = B3Geo<G>;
  constexpr int g = I / B3Steps<G>::SPG, r = I % B3Steps<G>::SPG;
  constexpr int t = g * Gm::CPG + 5 * r;   // first chunk of the step
  if constexpr (r < Gm::Q) {
    D0 = mfma_chunk<t + 0>(R.a, u2_t{e[0].x, e[0].y}, D0);
    D1 = mfma_chunk<t + 1>(R.a, u2_t{e[1].x, e[1].y}, D1);
    D0 = mfma_chunk<t + 2>(R.a, u2_t{e[2].x, e[2].y}, D0);
    D1 = mfma_chunk<t + 3>(R.a, u2_t{e[3].x, e[3].y}, D1);
    D0 = mfma_chunk<t + 4>(R.a, u2_t{e[0].z | e[1].w, e[2].z | e[3].w}, D0);
  } else if constexpr (Gm::T == 2) {
    D1 = mfma_chunk<t + 0>(R.a, u2_t{e[0].x, e[0].y}, D1);
    D0 = mfma_chunk<t + 1>(R.a, u2_t{e[1].x, e[1].y}, D0);
    if constexpr (Gm::T4) D1 = mfma_chunk<t + 2>(R.a, u2_t{e[0].z | e[1].w, 0u}, D1);
  } else {
    static_assert(Gm::T == 1, "tails of one or two bytes");
    D1 = mfma_chunk<t + 0>(R.a, u2_t{e[0].x, e[0].y}, D1);
    if constexpr (Gm::T4) D0 = mfma_chunk<t + 1>(R.a, u2_t{e[0].z, 0u}, D0);
  }
}

template <int G, int MT>
__device__ __forceinline__ void b3_stage_full(const uint8_t* lds, uint32_t coff, const uint32_t (&W)[kStageBytes / 4],
                                              StageRegs<G>& R, const u4_t (&SC)[B3Geo<G>::SCW], float (&acc)[MT]) {
  using Gm = B3Geo<G>;
  constexpr int P = TERN_B3_DEPTH;
  constexpr int NS = B3Steps<G>::NS, SPG = B3Steps<G>::SPG;
  u4_t E[P + 1][4];
  f4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
  sfor<0, P>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i < NS) b3_load_step<G, i>(lds, coff, W, E[i % (P + 1)]);
  });
  sfor<0, NS>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i + P < NS) b3_load_step<G, i + P>(lds, coff, W, E[(i + P) % (P + 1)]);
    b3_mfma_step<G, i>(R, E[i % (P + 1)], D0, D1);
    // chunks [tf, tl] of this step; refill the registers whose last chunk is among them
    constexpr int g = i / SPG, r = i % SPG;
    constexpr int tf = g * Gm::CPG + 5 * r;
    constexpr int tl = r < Gm::Q ? tf + 4 : g * Gm::CPG + Gm::CPG - 1;
    sfor<0, Gm::AREG>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int last = 16 * u + 15 < Gm::CPS ? 16 * u + 15 : Gm::CPS - 1;
      if constexpr (last >= tf && last <= tl) R.a[u] = load_areg(R, R.next + 128u * u);
    });
    if constexpr (r == SPG - 1) {
      const uint32_t sw = SC[g / 8][(g % 8) / 2];
      const float sc = h2f((uint16_t)(g % 2 ? sw >> 16 : sw & 0xFFFFu));
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = fmaf(sc, D0[m] + D1[m], acc[m]);
      D0 = f4_t{0.f, 0.f, 0.f, 0.f};
      D1 = f4_t{0.f, 0.f, 0.f, 0.f};
    }
  });
}

// Residual pass: the residual planes and the offset of kB3ResRows rows of
// one product, summed in FP32 into its rsum before the plane-0 product runs
// (which adds them when it writes y).  The activations are staged in LDS a
// window of groups at a time, each group padded by 16 bytes (lanes that read
// different groups then use different banks); entries (one per thread) are
// decoded from their 2-bit blocks and multiplied against them; each row's
// thread then adds its entries' values in entry order, window by window, so
// the sum is in (row, group) order.  Offsets use FP32 group sums of x taken
// from the staged windows.  Runs with several workgroups per CU, so the
// latency of its gathers hides behind other workgroups.
constexpr int kResThreads = kB3ResRows;
constexpr int kResPer = 4;            // entries per thread and chunk
constexpr int kResChunk = kResPer * kResThreads;
constexpr int kResBatch = 4;          // activation loads per thread in flight while staging

// Activation window of a launch whose longest product has max_k inputs,
// within lds_cap bytes of LDS in all: every group when they fit, else the
// most whole groups that do.
template <int G, int MT>
constexpr int res_window(int max_k, int lds_cap) {
  const int per = MT * (2 * G + 16);
  const int room = lds_cap - kResChunk * MT * 4 - MT * (max_k / G) * 4;
  return (max_k / G) * per <= room ? (max_k / G) * per : room / per * per;
}
template <int G, int MT>
constexpr int res_lds_bytes(int max_k, int lds_cap) {
  return res_window<G, MT>(max_k, lds_cap) + kResChunk * MT * 4 + MT * (max_k / G) * 4;
}

// TABLE: units and descriptors from device tables; else the row blocks of
// `one` (a compile-time choice: a descriptor chosen at run time between a
// table and the argument would be copied to scratch memory)
template <int G, int MT, bool TABLE>
__global__ __launch_bounds__(kResThreads) void b3_res_kernel(const GemvDesc* __restrict__ descs,
                                                             const B3ResItem* __restrict__ units, GemvDesc one,
                                                             int window, int nunits,
                                                             const B3Prep* __restrict__ preps, int prep_bx) {
  constexpr int GP = 2 * G + 16;
  constexpr int CPGX = 2 * G / 16;
  if constexpr (TABLE) {
    // workgroups past the units prepare the activation layouts of the
    // product launch that follows (one launch less)
    if ((int)blockIdx.x >= nunits) {
      const int pb = (int)blockIdx.x - nunits, by = pb / prep_bx;
      const B3Prep p = preps[by / MT];
      b3_prep_rows<G>(p, pb % prep_bx, by % MT);
      return;
    }
  }
  extern __shared__ uint4 res_smem[];
  uint8_t* xw = reinterpret_cast<uint8_t*>(res_smem);
  float* vals = reinterpret_cast<float*>(xw + window);
  GemvDesc d;
  int rb, slot;
  uint32_t ua0 = 0, ua1 = 0;
  if constexpr (TABLE) {
    const B3ResItem u = units[blockIdx.x];
    d = descs[u.desc];
    rb = (int)u.rb;
    slot = (int)u.slot;
    ua0 = u.a0;
    ua1 = u.a1;
  } else {
    d = one;
    rb = (int)blockIdx.x / d.rslots;
    slot = (int)blockIdx.x % d.rslots;
  }
  // this unit's residual plane (-1: none, the offset alone) and entry range
  // of the row block; slot 0 also adds the offset
  const int rplane = d.planes > 1 ? slot / d.rsplit : -1;
  const int rpart_ix = d.planes > 1 ? slot % d.rsplit : 0;
  const bool with_off = d.offset_mode != 0 && slot == 0;
  float* xsum = vals + kResChunk * MT;
  const int tid = threadIdx.x;
  const int r0 = rb * kB3ResRows;
  const int rlast = min(r0 + kB3ResRows, d.n);
  const int row = r0 + tid;
  const bool row_ok = row < rlast;
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;
  const int wgn = min(d.ng, window / (MT * GP));

  // a chunk of entries [c0, c1) of a plane: every load first (thread tid
  // takes entries c0 + tid + r * kResThreads)
  uint32_t gi[kResPer];
  u4_t bv[kResPer][G / 64];
  auto load_chunk = [&](const GLOBAL uint32_t* gidx, const GLOBAL u4_t* blocks, uint32_t c0, uint32_t c1) {
#pragma unroll
    for (int r = 0; r < kResPer; ++r) {
      const uint32_t e = c0 + (uint32_t)(tid + r * kResThreads);
      gi[r] = e < c1 ? gidx[e] : 0xFFFFu;
#pragma unroll
      for (int q = 0; q < G / 64; ++q)
        bv[r][q] = e < c1 ? __builtin_nontemporal_load(blocks + (size_t)e * (G / 64) + q) : u4_t{0u, 0u, 0u, 0u};
    }
  };
  // the plane's entries of the row block, [E0, E1), and this unit's part
  // [A0, A1) of them; (selects, not indexing with the plane: the descriptor
  // stays in registers)
  const GLOBAL uint32_t* rowptr = gp(rplane == 1 ? d.rowptr[1] : d.rowptr[0]);
  const GLOBAL uint32_t* gidx = gp(rplane == 1 ? d.gidx[1] : d.gidx[0]);
  const GLOBAL u4_t* blocks = reinterpret_cast<const GLOBAL u4_t*>(gp(rplane == 1 ? d.blocks[1] : d.blocks[0]));
  uint32_t A0 = 0, A1 = 0, rp_lo = 0, rp_hi = 0;
  if (rplane >= 0) {
    if constexpr (TABLE) {  // prepared with the table (launch_b3_res_ranges)
      A0 = ua0;
      A1 = ua1;
    } else {
      const uint32_t E0 = rowptr[r0], E1 = rowptr[rlast];
      const uint64_t len = E1 - E0;
      A0 = E0 + (uint32_t)(len * (uint64_t)rpart_ix / (uint64_t)d.rsplit);
      A1 = E0 + (uint32_t)(len * (uint64_t)(rpart_ix + 1) / (uint64_t)d.rsplit);
    }
    rp_lo = row_ok ? rowptr[row] : 0u;
    rp_hi = row_ok ? rowptr[row + 1] : 0u;
  }
  // the first chunk is requested before the activations are staged, so that
  // the two latencies overlap
  bool prefetched = false;
  if (A0 < A1) {
    load_chunk(gidx, blocks, A0, min(A1, A0 + (uint32_t)kResChunk));
    prefetched = true;
  }

  // (a unit with neither entries nor the offset stages nothing)
  for (int wg0 = 0; wg0 < (with_off || A0 < A1 ? d.ng : 0); wg0 += wgn) {
    const int wg1 = min(d.ng, wg0 + wgn), wn = wg1 - wg0;
    __syncthreads();  // the previous window is no longer read
    // stage the window: kResBatch loads per thread in flight, then the stores
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const GLOBAL uint8_t* xsrc =
          reinterpret_cast<const GLOBAL uint8_t*>(gp(d.x)) + ((size_t)min(m, d.m - 1) * d.k + (size_t)wg0 * G) * 2;
      const int total = wn * CPGX;
      for (int cb = 0; cb < total; cb += kResThreads * kResBatch) {
        u4_t v[kResBatch];
#pragma unroll
        for (int j = 0; j < kResBatch; ++j) {
          const int c = cb + tid + j * kResThreads;
          if (c < total) v[j] = *reinterpret_cast<const GLOBAL u4_t*>(xsrc + (size_t)c * 16);
        }
#pragma unroll
        for (int j = 0; j < kResBatch; ++j) {
          const int c = cb + tid + j * kResThreads;
          if (c < total) *reinterpret_cast<u4_t*>(xw + (m * wgn + c / CPGX) * GP + 16 * (c % CPGX)) = v[j];
        }
      }
    }
    __syncthreads();
    if (with_off) {  // group sums of x, in position order
      for (int c = tid; c < MT * wn; c += kResThreads) {
        const int m = c / wn, gl = c % wn;
        const uint32_t* xg = reinterpret_cast<const uint32_t*>(xw + (m * wgn + gl) * GP);
        float sx = 0.f;
        for (int i = 0; i < G / 2; ++i) {
          sx += h2f((uint16_t)(xg[i] & 0xFFFFu));
          sx += h2f((uint16_t)(xg[i] >> 16));
        }
        xsum[m * d.ng + wg0 + gl] = sx;
      }
    }
    {
      for (uint32_t c0 = A0; c0 < A1; c0 += kResChunk) {
        const uint32_t c1 = min(A1, c0 + (uint32_t)kResChunk);
        if (prefetched) prefetched = false;  // (the first chunk, in the first window)
        else load_chunk(gidx, blocks, c0, c1);
#pragma unroll
        for (int r = 0; r < kResPer; ++r) {
          const int g = (int)(gi[r] & 0xFFFFu);
          float part[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) part[m] = 0.f;
          if (g >= wg0 && g < wg1) {
#pragma unroll
            for (int q = 0; q < G / 64; ++q) {
              const uint32_t ws[4] = {bv[r][q].x, bv[r][q].y, bv[r][q].z, bv[r][q].w};
#pragma unroll
              for (int m = 0; m < MT; ++m) {
                const uint8_t* xg = xw + (m * wgn + (g - wg0)) * GP + q * 128;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                  const u4_t x0 = *reinterpret_cast<const u4_t*>(xg + 32 * u);
                  const u4_t x1 = *reinterpret_cast<const u4_t*>(xg + 32 * u + 16);
                  const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                  for (int i = 0; i < 8; ++i) part[m] = dot2(pair_of(ws[u], 14 - 2 * i), xs[i], part[m]);
                }
              }
            }
            const float rs = 0.5f * h2f((uint16_t)(gi[r] >> 16));
#pragma unroll
            for (int m = 0; m < MT; ++m) part[m] *= rs;
          }
          const uint32_t e = c0 + (uint32_t)(tid + r * kResThreads);
          if (e < c1) {
#pragma unroll
            for (int m = 0; m < MT; ++m) vals[(e - c0) * MT + m] = part[m];
          }
        }
        __syncthreads();
        // this row's entries of the chunk, in entry order (entries outside
        // the window add an exact zero)
        const uint32_t lo = max(rp_lo, c0), hi = min(rp_hi, c1);
        for (uint32_t e = lo; e < hi; ++e)
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[m] += vals[(e - c0) * MT + m];
        __syncthreads();
      }
    }
  }
  __syncthreads();  // the group sums are complete
  if (with_off && row_ok) {
    const GLOBAL uint16_t* off = gp(d.offset);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (d.offset_mode == 1) {
        float sx = 0.f;
        for (int g = 0; g < d.ng; ++g) sx += xsum[m * d.ng + g];
        acc[m] = fmaf(h2f(off[row]), sx, acc[m]);
      } else {
        for (int g = 0; g < d.ng; ++g) acc[m] = fmaf(h2f(off[(size_t)row * d.ng + g]), xsum[m * d.ng + g], acc[m]);
      }
    }
  }
  float* rs = const_cast<float*>(d.rsum);
  if (d.rslots > 1) {
    // this unit's sums; the row block's last unit adds them in slot order
    if (row_ok) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < d.m) part_store(d.rpart + ((size_t)slot * d.m + m) * d.n + row, acc[m]);
    }
    if (!last_part(d.rctr + rb, d.rslots)) return;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      acc[m] = 0.f;
      if (m < d.m && row_ok)
        for (int sl = 0; sl < d.rslots; ++sl) acc[m] += part_load(d.rpart + ((size_t)sl * d.m + m) * d.n + row);
    }
  }
  if (row_ok) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < d.m) rs[(size_t)m * d.n + row] = acc[m];
  }
}

template <int G, int MT, bool TABLE>
__global__ __launch_bounds__(kB3Threads) void gemv_b3_kernel(const GemvDesc* __restrict__ descs,
                                                             const B3Item* __restrict__ items,
                                                             uint32_t* __restrict__ queue, GemvDesc one,
                                                             int nitems) {
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
  const uint32_t coff = (uint32_t)(lane % kLutCopies) * 16u;
  // Items.  With a table: one queue per XCD (workgroups are dealt to the
  // XCDs in turn), each a list of items in decreasing cost; wavefront w of
  // the queue's workgroups starts with its item w and takes further ones from
  // the queue's counter, so that wavefronts that run faster (the older wave of
  // a SIMD wins issue, CUs differ in speed) take more items.  Without a table
  // wavefront w takes items w, w + W, ... of the one descriptor.
  int gw = (int)blockIdx.x * kB3Waves + wave;
  int nw = (int)gridDim.x * kB3Waves;
  int ibeg = 0, iend = nitems;
  uint32_t* qc = queue;
  if constexpr (TABLE) {
    const int q = (int)blockIdx.x % kB3Queues;
    qc = queue + q * kB3QueueWords;
    ibeg = (int)qc[2];
    iend = (int)qc[3];
    gw = ((int)blockIdx.x / kB3Queues) * kB3Waves + wave;
    nw = (((int)gridDim.x - q + kB3Queues - 1) / kB3Queues) * kB3Waves;
  }
  int next = 0;
  for (int it = ibeg + gw; it < iend; it = next) {
    uint32_t qv = 0;
    GemvDesc d;
    int rb, part;
    if constexpr (TABLE) {
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
    const int gb = min(d.ng, s1 * Gm::SG);
    // the residual planes' and offset's sums of the lane's row (residual
    // pass), requested before the stream so that no later wait holds on it
    float rres[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
      rres[m] = d.rsum && row_ok ? d.rsum[(size_t)min(m, d.m - 1) * d.n + row] : 0.f;

    const __amdgpu_buffer_rsrc_t rw = rsrc(d.plane0 + (size_t)row0 * d.stride, (size_t)(d.n - row0) * d.stride);
    const __amdgpu_buffer_rsrc_t rs = rsrc(d.scale0 + (size_t)row0 * d.ng, (size_t)(d.n - row0) * d.ng * 2);
    const size_t x5row = (size_t)d.ng * Gm::CPG * 8;   // bytes per activation row of x5
    const __amdgpu_buffer_rsrc_t rx = rsrc(d.x5, x5row * d.m);
    const uint32_t svoff = (uint32_t)lane * (uint32_t)d.ng * 2u;
    const uint32_t avoff = (uint32_t)min(lane % 4, d.m - 1) * (uint32_t)x5row + (uint32_t)(lane / 4) * 8u;

    // the lane's share of a stage's loads: chunk 64 u + lane = (row, 16-byte
    // column), computed per item (the opaque copy of the lane index keeps the
    // compiler from holding the lane-only parts for the whole launch)
    int lq = lane;
    asm volatile("" : "+v"(lq));
    uint32_t voff[kStageChunks];
#pragma unroll
    for (int u = 0; u < kStageChunks; ++u) {
      const int c = 64 * u + lq;
      voff[u] = (uint32_t)(c / kStageChunks) * (uint32_t)d.stride + (uint32_t)(c % kStageChunks) * 16u;
    }
    // stage s into the LDS buffer and its scales into SC
    auto issue = [&](int s, u4_t (&SC)[Gm::SCW]) {
#pragma unroll
      for (int u = 0; u < kStageChunks; ++u) lds_load16(rw, buf + 1024 * u, voff[u] + (uint32_t)s * kStageBytes);
      // scales: 16-byte loads when every row's scales start on a dword (an
      // unaligned dword that straddles the end of the array would read as
      // zero); one load per scale otherwise
      if ((d.ng & 1) == 0) {
#pragma unroll
        for (int w = 0; w < Gm::SCW; ++w)
          SC[w] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, svoff + (uint32_t)(s * Gm::SG) * 2u + 16u * w, 0, 0));
      } else {
#pragma unroll
        for (int w = 0; w < Gm::SCW; ++w) {
          uint32_t h[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            h[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, svoff + (uint32_t)(s * Gm::SG + 8 * w + j) * 2u, 0, 0);
          SC[w] = u4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
      }
    };

    float acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = 0.f;

    StageRegs<G> R;
    R.rx = rx;
    auto body = [&](int s, const u4_t (&SCc)[Gm::SCW], u4_t (&SCn)[Gm::SCW]) {
      // stage s is in LDS and its scales have arrived: everything but the
      // AREG activation loads issued after them (this stage's registers,
      // which the compiler waits for at their first use)
      wait_vm<Gm::AREG>();
      wave_sync();
      uint32_t W[kStageBytes / 4];
#pragma unroll
      for (int q = 0; q < kStageChunks; ++q) {
        const u4_t v = *reinterpret_cast<const u4_t*>(buf + lane * kStageBytes + 16 * q);
        W[4 * q] = v.x; W[4 * q + 1] = v.y; W[4 * q + 2] = v.z; W[4 * q + 3] = v.w;
      }
      wait_lgkm0();  // the buffer is free for the next stage
      wave_sync();
      if (s + 1 < s1) {
        issue(s + 1, SCn);
      } else if constexpr (TABLE) {
        // the next item, requested during the last stage: vector memory
        // operations complete in order, so a request issued before a
        // stage's loads would hold up the wait for them
        if (lane == 0) qv = __hip_atomic_fetch_add(qc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      R.next = avoff + (uint32_t)((s + 1) * Gm::CPS) * 8u;
      const int gs = s * Gm::SG;
      if (gs + Gm::SG <= gb) {
        b3_stage_full<G, MT>(lds, coff, W, R, SCc, acc);
      } else {  // the row's last, partial stage (no next stage)
        sfor<0, Gm::SG>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          if (gs + g < gb) b3_group<G, MT, g>(lds, coff, W, R, SCc, acc);
        });
      }
    };

    if (s0 < s1) {
      u4_t SA[Gm::SCW], SB[Gm::SCW];
      wait_lgkm0();
      wave_sync();
      issue(s0, SA);
#pragma unroll
      for (int u = 0; u < Gm::AREG; ++u) R.a[u] = load_areg(R, avoff + (uint32_t)(s0 * Gm::CPS) * 8u + 128u * u);
      int s = s0;
      for (; s + 1 < s1; s += 2) {
        body(s, SA, SB);
        body(s + 1, SB, SA);
      }
      if (s < s1) body(s, SA, SB);
    } else if constexpr (TABLE) {
      if (lane == 0) qv = __hip_atomic_fetch_add(qc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    wave_sync();
    if constexpr (TABLE) next = ibeg + nw + (int)__builtin_amdgcn_readfirstlane(qv);
    else next = it + nw;
    // the residual sums join the first K part (or the whole row)
    if (part == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] += rres[m];
    }

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
  if constexpr (TABLE) {
    // the last wavefront to finish (every fetch from the queue has returned
    // by then) clears the queue for the next launch
    if (lane == 0) {
      const uint32_t done = __hip_atomic_fetch_add(qc + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done == (uint32_t)nw - 1u) {
        __hip_atomic_store(qc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(qc + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int G, int MT>
hipError_t launch_b3_mt(const GemvDesc* descs, const B3Item* items, uint32_t* queue, int nwg, const GemvDesc& one,
                        int nitems, hipStream_t s) {
  if (descs)
    hipLaunchKernelGGL((gemv_b3_kernel<G, MT, true>), dim3(nwg), dim3(kB3Threads), 0, s, descs, items, queue, one,
                       nitems);
  else
    hipLaunchKernelGGL((gemv_b3_kernel<G, MT, false>), dim3(nwg), dim3(kB3Threads), 0, s, descs, items, queue, one,
                       nitems);
  return hipGetLastError();
}

template <int G>
hipError_t launch_b3_g(int mt, const GemvDesc* descs, const B3Item* items, uint32_t* queue, int nwg,
                       const GemvDesc& one, int nitems, hipStream_t s) {
  switch (mt) {
    case 1: return launch_b3_mt<G, 1>(descs, items, queue, nwg, one, nitems, s);
    case 2: return launch_b3_mt<G, 2>(descs, items, queue, nwg, one, nitems, s);
    case 4: return launch_b3_mt<G, 4>(descs, items, queue, nwg, one, nitems, s);
    default: return hipErrorInvalidValue;
  }
}

template <int G, int MT>
hipError_t launch_res_mt(const GemvDesc* descs, const B3ResItem* units, int nunits, const GemvDesc& one, int max_k,
                         int lds_cap, const B3Prep* preps, int nprep, int prep_max_k, hipStream_t s) {
  const int window = res_window<G, MT>(max_k, lds_cap);
  if (window < MT * (2 * G + 16)) return hipErrorInvalidValue;  // not one group fits
  const size_t lds = (size_t)res_lds_bytes<G, MT>(max_k, lds_cap);
  if (units) {
    const int prep_bx = std::max(1, (prep_max_k / G * B3Geo<G>::CPG + 255) / 256);
    // one block row per activation row of the launch (MT >= m): at m = 1 the
    // 8B-class stack's launch held 6,480 empty workgroups with four
    // (stack 406.3-406.5 against 407.9-408.1 us per token)
    const int prep_blocks = preps ? prep_bx * nprep * MT : 0;
    hipLaunchKernelGGL((b3_res_kernel<G, MT, true>), dim3(nunits + prep_blocks), dim3(kResThreads), lds, s, descs,
                       units, one, window, nunits, preps, prep_bx);
  } else {
    hipLaunchKernelGGL((b3_res_kernel<G, MT, false>), dim3(nunits), dim3(kResThreads), lds, s, descs, units, one,
                       window, nunits, preps, 1);
  }
  return hipGetLastError();
}

template <int G>
hipError_t launch_res_g(int mt, const GemvDesc* descs, const B3ResItem* units, int nunits, const GemvDesc& one,
                        int max_k, int lds_cap, const B3Prep* preps, int nprep, int prep_max_k, hipStream_t s) {
  switch (mt) {
    case 1: return launch_res_mt<G, 1>(descs, units, nunits, one, max_k, lds_cap, preps, nprep, prep_max_k, s);
    case 2: return launch_res_mt<G, 2>(descs, units, nunits, one, max_k, lds_cap, preps, nprep, prep_max_k, s);
    case 4: return launch_res_mt<G, 4>(descs, units, nunits, one, max_k, lds_cap, preps, nprep, prep_max_k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int b3_res_window_groups(int group, int mt, int max_k, int lds_cap) {
  const int ng = max_k / group, per = mt * (2 * group + 16);
  const int room = lds_cap - kResChunk * mt * 4 - mt * ng * 4;
  return room <= 0 ? 0 : std::min(ng, room / per);
}

hipError_t launch_b3_res(int group, int mt, const GemvDesc* descs, const B3ResItem* units, int nunits,
                         const GemvDesc& one, int max_k, int lds_cap, const B3Prep* preps, int nprep, int prep_max_k,
                         hipStream_t s) {
  if (nunits <= 0) return hipSuccess;
  if (group == 64) return launch_res_g<64>(mt, descs, units, nunits, one, max_k, lds_cap, preps, nprep, prep_max_k, s);
  if (group == 128) return launch_res_g<128>(mt, descs, units, nunits, one, max_k, lds_cap, preps, nprep, prep_max_k, s);
  return hipErrorInvalidValue;
}

namespace {
// The entry range [a0, a1) of every residual-pass unit of a table: its part
// of its plane's entries of its row block.
__global__ __launch_bounds__(256) void b3_res_ranges_kernel(const GemvDesc* __restrict__ descs,
                                                            B3ResItem* __restrict__ units, int nunits) {
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (i >= nunits) return;
  B3ResItem u = units[i];
  const GemvDesc& d = descs[u.desc];
  u.a0 = u.a1 = 0u;
  if (d.planes > 1) {
    const int rplane = (int)u.slot / d.rsplit, part = (int)u.slot % d.rsplit;
    const uint32_t* rowptr = rplane == 1 ? d.rowptr[1] : d.rowptr[0];
    const int r0 = (int)u.rb * kB3ResRows, rlast = min(r0 + kB3ResRows, d.n);
    const uint32_t E0 = rowptr[r0], E1 = rowptr[rlast];
    const uint64_t len = E1 - E0;
    u.a0 = E0 + (uint32_t)(len * (uint64_t)part / (uint64_t)d.rsplit);
    u.a1 = E0 + (uint32_t)(len * (uint64_t)(part + 1) / (uint64_t)d.rsplit);
  }
  units[i] = u;
}
}  // namespace

hipError_t launch_b3_res_ranges(const GemvDesc* descs, B3ResItem* units, int nunits, hipStream_t s) {
  if (nunits <= 0) return hipSuccess;
  hipLaunchKernelGGL(b3_res_ranges_kernel, dim3((nunits + 255) / 256), dim3(256), 0, s, descs, units, nunits);
  return hipGetLastError();
}

int b3_chunks_per_group(int group) { return group == 64 ? B3Geo<64>::CPG : B3Geo<128>::CPG; }
int b3_stage_groups(int group) { return group == 64 ? B3Geo<64>::SG : B3Geo<128>::SG; }

hipError_t launch_b3_prep(int group, const B3Prep* preps, int count, const B3Prep& one, int max_k, hipStream_t s) {
  const int rows = (preps ? count : 1) * 4;
  if (rows <= 0 || max_k <= 0) return hipSuccess;
  const int chunks = max_k / group * b3_chunks_per_group(group);
  const dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)rows);
  if (group == 64) hipLaunchKernelGGL(b3_prep_kernel<64>, grid, dim3(256), 0, s, preps, one);
  else if (group == 128) hipLaunchKernelGGL(b3_prep_kernel<128>, grid, dim3(256), 0, s, preps, one);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_b3_prep_rot(int group, int block, const B3Prep* preps, int count, int max_k, hipStream_t s) {
  if (count <= 0 || max_k <= 0) return hipSuccess;
  const int span = std::max(group, block);
  const dim3 grid((unsigned)((max_k + span - 1) / span), (unsigned)count);
  if (group == 128 && block == 128) hipLaunchKernelGGL((b3_prep_rot_kernel<128, 128>), grid, dim3(256), 0, s, preps);
  else if (group == 128 && block == 64) hipLaunchKernelGGL((b3_prep_rot_kernel<128, 64>), grid, dim3(256), 0, s, preps);
  else if (group == 64 && block == 128) hipLaunchKernelGGL((b3_prep_rot_kernel<64, 128>), grid, dim3(256), 0, s, preps);
  else if (group == 64 && block == 64) hipLaunchKernelGGL((b3_prep_rot_kernel<64, 64>), grid, dim3(256), 0, s, preps);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemv_b3(int group, int mt, const GemvDesc* descs, const B3Item* items, uint32_t* queue, int nwg,
                          const GemvDesc& one, int nitems, hipStream_t s) {
  if (nwg <= 0) return hipSuccess;
  if (group == 64) return launch_b3_g<64>(mt, descs, items, queue, nwg, one, nitems, s);
  if (group == 128) return launch_b3_g<128>(mt, descs, items, queue, nwg, one, nitems, s);
  return hipErrorInvalidValue;
}

}  // namespace tern
