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
#include <cstring>

#include "internal.h"
#include "kparts.h"

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
constexpr int kMaxBlocks = 12;     // blocks per wavefront
#ifndef TERN_MFMA_DEPTH
#define TERN_MFMA_DEPTH 2
#endif
constexpr int kDepth = TERN_MFMA_DEPTH;  // weight blocks a wavefront keeps in flight
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
// One 64-bit shift serves both words (a full-rate instruction on this GPU;
// the compiler would otherwise split it into two 32-bit ones): the high word
// picks up bits of w0 only below bit 14, which the mask clears.
template <int SH>
__device__ __forceinline__ uint64_t shl64(uint64_t v) {
  uint64_t r;
  asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "n"(SH), "v"(v));
  return r;
}

__device__ __forceinline__ void decode_two(uint32_t w0, uint32_t w1, h8_t* b) {
  const uint64_t wd = ((uint64_t)w1 << 32) | w0;
  u4_t lo[2], hi[2];
#define TERN_PAIR(P)                                                                          \
  do {                                                                                        \
    const uint64_t s_ = (P) == 7 ? wd : shl64<14 - 2 * (P)>(wd);                              \
    lo[(P) / 4][(P) % 4] = (uint32_t)s_ & 0xC000C000u;                                        \
    hi[(P) / 4][(P) % 4] = (uint32_t)(s_ >> 32) & 0xC000C000u;                                \
  } while (0)
  TERN_PAIR(0); TERN_PAIR(1); TERN_PAIR(2); TERN_PAIR(3);
  TERN_PAIR(4); TERN_PAIR(5); TERN_PAIR(6); TERN_PAIR(7);
#undef TERN_PAIR
  b[0] = __builtin_bit_cast(h8_t, lo[0]);
  b[1] = __builtin_bit_cast(h8_t, lo[1]);
  b[2] = __builtin_bit_cast(h8_t, hi[0]);
  b[3] = __builtin_bit_cast(h8_t, hi[1]);
}

__device__ __forceinline__ h8_t lds_h8(const uint8_t* lds, uint32_t off) {
  return *reinterpret_cast<const h8_t*>(lds + off);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes (64 trits) of block c (wave-uniform) of this lane's part of its
// row: a buffer resource from the item's first row (uniform), the lane's
// row and quarter as the per-lane offset and the block as the scalar one;
// bytes past the matrix read as zero.
__device__ __forceinline__ u4_t wload(__amdgpu_buffer_rsrc_t part, int c, uint32_t lane_off) {
  // c is the same in every lane (the compiler cannot prove it of values
  // derived from the wavefront index, and would loop over its values)
  return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(part, lane_off,
                                                                        __builtin_amdgcn_readfirstlane(c) * 64, 0));
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


// 16 bytes per lane from a buffer straight into LDS, without registers: lane
// l of the wavefront writes dst + 16 l, so dst must be the same in every lane
// (the chunk of the wavefront's first lane).  Counted by vmcnt like a load.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(n) alone (expcnt and lgkmcnt left free), n <= 63.
#define TERN_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

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
// Wavefronts per SIMD the kernel's registers are sized for (at least).
template <int G, int MP>
constexpr int mfma_waves_per_eu() { return MP == 8 || (G == 64 && MP == 4) ? 2 : 3; }

// ---- the rotation folded into the launch (RotFold): xr = blockdiag(R) x
// ("Post-Training Ternarization of Qwen3-4B", §4.2: inference rotates the
// activations into the basis the weights were quantized in).  Share s of
// an input covers kRotShareRows consecutive positions: LPR adjacent lanes
// form one position's row of R times x (each a 1/LPR part of the row, B /
// (2 LPR) FP16 pairs with v_dot2_f32_f16 in order), add their parts (lane
// distance 1, 2, ...: a fixed order, so runs are reproducible), and each
// even position stores itself and the next as one word.
template <int RBLK>
__device__ __forceinline__ void rot_share(const RotFold& f, int share) {
  constexpr int LPR = kThreads / kRotShareRows;  // lanes per position
  constexpr int CPT = RBLK / 8 / LPR;            // 16-byte chunks of a row per lane
  static_assert(LPR >= 1 && LPR <= 32 && CPT >= 1 && kThreads == LPR * kRotShareRows, "share shape");
  const RotBatch& a = f.a;
  // this share's input, picked with uniform selects (an indexed read would
  // copy the argument block to scratch memory)
  const uint16_t* R = a.R[0];
  const uint16_t* x = a.x[0];
  uint16_t* out = a.out[0];
  int k = a.k[0], first = 0;
#pragma unroll
  for (int q = 1; q < kMaxRotations; ++q)
    if (q < a.count && share >= a.begin[q]) {
      R = a.R[q];
      x = a.x[q];
      out = a.out[q];
      k = a.k[q];
      first = a.begin[q];
    }
  const int t = threadIdx.x, i = t / LPR, j = t % LPR;
  const int pos = (share - first) * kRotShareRows + i;  // the last share of an input may pass k
  const bool live = pos < k;
  const int pc = live ? pos : k - 1;
  const int b = pc / RBLK, ib = pc % RBLK;
  const GLOBAL u4_t* rr = reinterpret_cast<const GLOBAL u4_t*>(gp(R) + ((size_t)b * RBLK + ib) * RBLK) + j * CPT;
  u4_t rv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) rv[c] = rr[c];
  for (int m = 0; m < a.m; ++m) {
    const GLOBAL u4_t* xp = reinterpret_cast<const GLOBAL u4_t*>(gp(x) + (size_t)m * k + (size_t)b * RBLK) + j * CPT;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const u4_t xv = xp[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // through plain words: a bit cast of a vector element itself reads
        // element 0 with this compiler
        const uint32_t rw = rv[c][e], xw = xv[e];
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, rw), __builtin_bit_cast(h2_t, xw), acc, false);
      }
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, kWave);
    const float next = __shfl_down(acc, LPR, kWave);  // position pos + 1
    if (live && t % (2 * LPR) == 0) {
      const uint32_t word = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)acc) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)next) << 16);
      __hip_atomic_store(reinterpret_cast<uint32_t*>(out + (size_t)m * k + pos), word, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the stores are acknowledged by the device-coherent level, in every
  // wavefront, before the share counts itself in.  Two levels: share s
  // counts itself in at sub-count s % kRotSubs; the share that completes a
  // sub-count clears it (no other share of this launch touches it again)
  // and counts the sub-count in at the top count; the share that completes
  // the top count raises the ready flag copy of every group that has members
  // (one per lane of wavefront 0; a group with none would never lower it).
  // Returning atomics on one word are served one at a time, so this keeps
  // each chain short (about shares / kRotSubs, then kRotSubs) instead of
  // one chain of every share.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (t < kWave) {
    uint32_t last = 0u;
    if (t == 0) {
      const int c = share % kRotSubs;
      const uint32_t members = (uint32_t)(f.shares / kRotSubs + (c < f.shares % kRotSubs ? 1 : 0));
      uint32_t* sub = f.sync + kRotLineWords * (1 + kRotFlags + c);
      if (__hip_atomic_fetch_add(sub, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == members) {
        __hip_atomic_store(sub, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t subs = (uint32_t)min(f.shares, kRotSubs);
        last = __hip_atomic_fetch_add(f.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == subs ? 1u : 0u;
      }
    }
    last = __shfl(last, 0, kWave);
    if (last && t < (int)gridDim.x - f.shares)
      __hip_atomic_store(f.sync + kRotLineWords * (1 + t), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The counters of a folded rotation, one 256-byte line each (RotFold.sync):
// line 0 holds the share sub-counts completed [0], the waiter groups done
// [1] and the give-up word [2]; line 1 + c holds copy c of the ready flag [0]
// and the count of group c's workgroups through the wait [1]; line
// 1 + kRotFlags + c holds share sub-count c [0].  A product workgroup
// belongs to group (its index) % kRotFlags, so every address is polled by a
// few workgroups only (accesses to one address are served one at a time).
static_assert(kRotFlags == kWave, "one flag copy per lane");

// Product side: wait until this group's flag copy is raised (bounded; a wait
// that gives up records it and goes on), then count the workgroup in at its
// group.  Returns that count's old value (thread 0; used by rot_release).
// Shares are the launch's lowest workgroups, so each is placed before any
// workgroup that waits for it, and shares never wait.
constexpr uint64_t kRotWaitTicks = 2000000;  // 20 ms of the 100 MHz clock
__device__ __forceinline__ uint32_t rot_wait(const RotFold& f, int wg) {
  uint32_t* line = f.sync + kRotLineWords * (1 + wg % kRotFlags);
  uint32_t mine = 0u;
  if (threadIdx.x == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      __builtin_amdgcn_s_sleep(2);
      if (__builtin_amdgcn_s_memrealtime() - t0 > kRotWaitTicks) {
        __hip_atomic_store(f.sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    mine = __hip_atomic_fetch_add(line + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return mine;
}

// Thread 0 of a product workgroup, late in its run (the count returned by
// rot_wait has arrived by then): the group's last workgroup lowers the
// group's flag copy and clears its count, then counts the group in; the
// last group clears line 0 for the next launch.
__device__ __forceinline__ void rot_release(const RotFold& f, int wg, uint32_t mine) {
  const int items = (int)gridDim.x - f.shares;
  const int c = wg % kRotFlags;
  const uint32_t members = (uint32_t)(items / kRotFlags + (c < items % kRotFlags ? 1 : 0));
  if (mine + 1u != members) return;
  uint32_t* line = f.sync + kRotLineWords * (1 + c);
  __hip_atomic_store(line, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(line + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t groups = (uint32_t)min(items, kRotFlags);
  if (__hip_atomic_fetch_add(f.sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == groups) {
    __hip_atomic_store(f.sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(f.sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The product; with RBLK > 0 the launch's first f.shares workgroups rotate
// (rot_share) and the activations are staged after rot_wait.
template <int G, int MP, int RBLK>
__device__ __forceinline__ void mfma_body(const GemvDesc* __restrict__ descs, const WgRec* __restrict__ recs,
                                          int ndesc, GemvDesc one, const RotFold& f) {
  if constexpr (RBLK > 0) {
    if ((int)blockIdx.x < f.shares) {
      rot_share<RBLK>(f, (int)blockIdx.x);
      return;
    }
  }
  const int wg = (int)blockIdx.x - (RBLK > 0 ? f.shares : 0);
  constexpr int GW = Win<MP>::GW;
  constexpr int NACC = Win<MP>::NACC;
  constexpr int GPB = kBlockTrits / G;      // groups per block
  constexpr int BW = GW / GPB;              // blocks per window
  static_assert(BW >= 1, "a window must hold at least one block");
  typedef typename ResQ<G>::T RB;
  extern __shared__ uint4 smem_all[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem_all);

  // grouped launches: this workgroup's record names its row range's
  // descriptor (a few per launch, so they stay in the L2) and its item;
  // otherwise the single descriptor
  GemvDesc d;
  int item;
  uint32_t te[5] = {0u, 0u, 0u, 0u, 0u};
  if (RBLK > 0 || ndesc > 0) {  // rotating launches are always grouped
    const WgRec rec = recs[wg];
    d = descs[rec.ri >> 20];
    item = (int)(rec.ri & 0xFFFFFu);
#pragma unroll
    for (int t = 0; t < 5; ++t) te[t] = rec.te[t];
  } else {
    d = one;
    item = wg - d.tile_begin;
  }
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
  const int row0 = d.row_base + rb * rw;
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

  // ---- 1. the small operands go straight into LDS (no registers), then
  // every wavefront requests its weights (below); the workgroup waits for the
  // small operands only, so the weight stream starts right after the
  // descriptor.  Scales, flat: 16-byte chunks covering this item's rows
  // (they are contiguous), from the 16-byte boundary at or below the first
  // scale; a chunk that reaches past the scale array goes through registers.
  const uintptr_t sfirst = (uintptr_t)(s0 + (size_t)row0 * d.ng);
  const uintptr_t sa0 = sfirst & ~(uintptr_t)15;
  const int sshift = (int)(sfirst - sa0) / 2;  // elements before row0's first scale
  const int nsch = sflat ? (int)(((uintptr_t)(s0 + (size_t)min(row0 + rw, d.n) * d.ng) - sa0 + 15) / 16) : 0;
  const uintptr_t send = (uintptr_t)(s0 + (size_t)d.n * d.ng);  // end of the scale array
  const int nsfull = min(nsch, (int)((send - sa0) / 16));       // chunks wholly inside it
  if (sflat) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(d.scale0, (uint32_t)(send - (uintptr_t)s0));
    const uint32_t sv0 = (uint32_t)(sa0 - (uintptr_t)s0);
    for (int u = 0; u * kThreads < nsfull; ++u)
      if (u * kThreads + tid < nsfull)
        lds_load16(rs, lds + scoff + (u * kThreads + wave * kWave) * 16, sv0 + (u * kThreads + tid) * 16);
  } else {
    // K split: the item's groups of each row (thread -> groups 32c + sgl, rows srr + 8u)
    uint16_t* ssm = reinterpret_cast<uint16_t*>(lds + scoff);
    const int sgl = tid % 32, srr = tid / 32;
    for (int c = 0; c * 32 < ngr; ++c) {
      const int g = c * 32 + sgl;
      if (g < ngr)
        for (int u = 0; u < rw / 8; ++u)
          ssm[(srr + 8 * u) * spitch + g] = s0[(size_t)min(row0 + srr + 8 * u, d.n - 1) * d.ng + ga + g];
    }
  }
  u4_t sfix = u4_t{0u, 0u, 0u, 0u};
  if (tid < nsch - nsfull) sfix = scale_chunk(s0, send, sa0 + (size_t)(nsfull + tid) * 16);
  // activations [dm][krp], row m at m * krp (chunk id at 16 id); zero past
  // the range.  Rotated activations are written during the launch, so they
  // are staged after rot_wait, with ordinary loads: the shares' stores went
  // through to the device-coherent level, and no workgroup reads the rotated
  // copy before the flag rises, so no L2 holds a line of it from before this
  // launch's stores (the L2s start each launch invalidated).
#define TERN_STAGE_X()                                                                        \
  do {                                                                                        \
    const __amdgpu_buffer_rsrc_t rx_ = rsrc(d.x, (uint32_t)dm * d.k * 2u);                    \
    for (int u = 0; u * kThreads < nx; ++u) {                                                 \
      const int id = u * kThreads + tid;                                                      \
      if (id < nx) {                                                                          \
        const int m = xrow_of<MP>(id, cpr);                                                   \
        const int kk = (id - m * cpr) * 8;                                                    \
        if (kk < kr) lds_load16(rx_, lds + xoff + (u * kThreads + wave * kWave) * 16, ((uint32_t)m * d.k + k0 + kk) * 2u); \
        else *reinterpret_cast<u4_t*>(lds + xoff + id * 16) = u4_t{0u, 0u, 0u, 0u};           \
      }                                                                                       \
    }                                                                                         \
  } while (0)
  if (RBLK == 0) TERN_STAGE_X();
  // first residual plane, when the plan indexed it and the item covers the
  // whole row: the workgroup's entries [e0, e1) (its rows are contiguous) are
  // staged in LDS with the other small operands -- their blocks as raw
  // 16-byte chunks and their index words (group | scale bits << 16)
  // (or, with an index per K part, the item's entries of every residual
  // plane in its K part)
  const bool part_idx = (RBLK > 0 || ndesc > 0) && d.pidx != nullptr;
  uint32_t e0 = 0, e1 = 0;
  if ((RBLK > 0 || ndesc > 0) && (part_idx || (d.gidx[0] != nullptr && sflat && d.planes == 2))) {
    const int nt = rw / kRowsWave;
    e0 = te[0];
    e1 = nt == 1 ? te[1] : nt == 2 ? te[2] : te[4];
  }
  const bool res_idx = e1 > e0 && e1 - e0 <= (uint32_t)kResStage;
  const uint32_t nres = res_idx ? e1 - e0 : 0u;
  constexpr int kBQ = G / 4 / 16;                          // 16-byte chunks per block
  const GLOBAL uint32_t* gix = gp(part_idx ? d.pidx : d.gidx[0]);
  const uintptr_t gfirst = (uintptr_t)(gix + e0), ga0 = gfirst & ~(uintptr_t)15;
  const int gshift = (int)(gfirst - ga0) / 4;
  const int nbch = (int)nres * kBQ;                        // block chunks
  const int ngch = res_idx ? (int)(((uintptr_t)(gix + e1) - ga0 + 15) / 16) : 0;  // index chunks
  if (res_idx) {
    // the index array sits in a 256-byte-rounded allocation of 16-byte aligned start
    const uint32_t nnz_ = part_idx ? d.pnnz : d.nnz[0];
    const __amdgpu_buffer_rsrc_t rb = rsrc(part_idx ? d.pblocks : d.blocks[0], nnz_ * (uint32_t)(G / 4));
    const __amdgpu_buffer_rsrc_t rg = rsrc(part_idx ? d.pidx : d.gidx[0], (nnz_ * 4u + 15u) & ~15u);
    for (int u = 0; u * kThreads < nbch; ++u)
      if (u * kThreads + tid < nbch)
        lds_load16(rb, lds + rstoff + (u * kThreads + wave * kWave) * 16, (e0 * kBQ + u * kThreads + tid) * 16u);
    const uint32_t gv0 = (uint32_t)(ga0 - (uintptr_t)gix);
    for (int u = 0; u * kThreads < ngch; ++u)
      if (u * kThreads + tid < ngch)
        lds_load16(rg, lds + rstoff + kResStage * (G / 4) + (u * kThreads + wave * kWave) * 16,
                   gv0 + (u * kThreads + tid) * 16u);
  }
  // this row's entries, for the sums
  uint32_t rp0 = 0, rp1 = 0;
  if (res_idx) {
    const GLOBAL uint32_t* rp_ = part_idx ? gp(d.prowptr) + (size_t)split * d.n : gp(d.rowptr[0]);
    rp0 = rp_[rowc];
    rp1 = rp_[rowc + 1];
  }

  // this wavefront's share of the staged entries (relative to e0): those of
  // its tile's rows, split evenly over the tile's kw wavefronts; their values
  // are computed between its plane-0 blocks and summed by this wavefront
  uint32_t we0 = 0, we1 = 0;
  if (res_idx) {
    const uint32_t tb = tile == 0 ? te[0] : tile == 1 ? te[1] : tile == 2 ? te[2] : te[3];
    const uint32_t tn = tile == 0 ? te[1] : tile == 1 ? te[2] : tile == 2 ? te[3] : te[4];
    const uint32_t ps = (tn - tb + kw - 1) / kw;
    we0 = min(tn, tb + kp * ps) - e0;
    we1 = min(tn, tb + (kp + 1) * ps) - e0;
  }
  const int nrb = (int)((we1 - we0 + 15u) / 16u);  // this wavefront's 16-entry batches
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
  const __amdgpu_buffer_rsrc_t wpart =
      rsrc(d.plane0 + (size_t)row0 * d.stride, (uint32_t)min((size_t)(d.n - row0) * d.stride, (size_t)0xFFFFFFF0u));
  const uint32_t wq = (uint32_t)(rowc - row0) * (uint32_t)d.stride + (uint32_t)(k0 + (nblk > 0 ? pb0 * kBlockTrits : 0)) / 4u +
                      (uint32_t)q * 16u;
  // the block (within each window) in which this lane's A slot is active:
  // slot r % GW holds group GPB * (block % BW) + q / (4 / GPB); -1 if never
  const int rg_ = (r % GW) - q / (4 / GPB);
  const int wsel = a_row && rg_ >= 0 && rg_ % GPB == 0 && rg_ / GPB < BW ? rg_ / GPB : -1;

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
  // batch J of this wavefront's share of the staged entries
#define TERN_RES_ONE(J)                                                                       \
  do {                                                                                        \
    const uint32_t b0_ = we0 + 16u * (uint32_t)(J);                                           \
    const uint32_t t_ = min(b0_ + r, we1 - 1);                                                \
    const RB bq_ = *reinterpret_cast<const RB*>(lds + rstoff + t_ * (G / 4) + q * sizeof(RB)); \
    const uint32_t gi_ = *reinterpret_cast<const uint32_t*>(lds + rstoff + kResStage * (G / 4) + (gshift + t_) * 4); \
    TERN_RES_BATCH(valr, b0_, we1, bq_, (int)(gi_ & 0xFFFFu), 0.5f * h2f((uint16_t)(gi_ >> 16))); \
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
    const uint32_t aoff_ = wsel == (I) % BW ? abase + (uint32_t)(C) * (kBlockTrits * 2) : 0u; \
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
    /* the weights, behind the small operands in every wavefront's queue */                  \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    constexpr int DP_ = NB < kDepth ? NB : kDepth;                                            \
    _Pragma("unroll") for (int i = 0; i < DP_; ++i) w_[i] = wload(wpart, min(i, max(nblk - 1, 0)), wq); \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    if (tid < nsch - nsfull) *reinterpret_cast<u4_t*>(lds + scoff + (nsfull + tid) * 16) = sfix; \
    if (tid < kZeroBytes / 16) *reinterpret_cast<u4_t*>(lds + tid * 16) = u4_t{0u, 0u, 0u, 0u}; \
    if (RBLK > 0) {                                                                           \
      /* the poll returns behind this wavefront's first DP_ blocks (loads */                  \
      /* complete in order), which arrive early; the rest stream after it */                  \
      rot_mine = rot_wait(f, wg);                                                             \
      TERN_STAGE_X();                                                                         \
      TERN_WAIT_VM(0);                                                                        \
    } else {                                                                                  \
      TERN_WAIT_VM(DP_); /* this wavefront's LDS loads have landed */                        \
    }                                                                                         \
    __syncthreads();                                                                          \
    /* plane 0, with this wavefront's residual batches after its first blocks */            \
    _Pragma("unroll") for (int i = 0; i < NB; ++i) {                                          \
      /* keep DP_ blocks in flight: request block i + DP_ before block i is used */          \
      if (i + DP_ < NB) w_[i + DP_] = wload(wpart, min(i + DP_, max(nblk - 1, 0)), wq);        \
      if (i < nblk) {                                                                         \
        TERN_BLOCK(w_[i], i, i);                                                              \
        if (i % BW == BW - 1) TERN_CLOSE(i / BW);                                             \
      }                                                                                       \
      if (i < nrb) TERN_RES_ONE(i);                                                           \
    }                                                                                         \
    if (nblk > 0 && nblk % BW != 0) TERN_CLOSE((nblk - 1) / BW);                              \
    for (int j_ = NB; j_ < nrb; ++j_) TERN_RES_ONE(j_);                                       \
  } while (0)
  uint32_t rot_mine = 0u;
  if (bpp > 8) TERN_BODY(kMaxBlocks);
  else TERN_BODY(8);
#undef TERN_BODY
#undef TERN_BLOCK
#undef TERN_CLOSE
#undef TERN_STAGE_X

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
    if (res_idx && (p == 0 || part_idx)) continue;  // staged: done with plane 0
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
#undef TERN_RES_ONE
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
  // staged residual entries of this row in this wavefront's share: the row's
  // four lanes take every fourth entry, then the quarters are added (fixed
  // order); the parts of a tile add their shares with the part sums below
  if (res_idx) {
    wave_sync();
    float rsum[MP];
#pragma unroll
    for (int m = 0; m < MP; ++m) rsum[m] = 0.f;
    if (row_ok) {
      const uint32_t lo = max(rp0 - e0, we0), hi = min(rp1 - e0, we1);
      for (uint32_t e = lo + q; e < hi; e += 4)
#pragma unroll
        for (int m = 0; m < MP; ++m) rsum[m] += valr[e * MP + m];
    }
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
  // ---- the parts of a row tile, summed in part order
  float* red = reinterpret_cast<float*>(lds + redoff);
  if (kw > 1) {
#pragma unroll
    for (int i = 0; i < NACC; ++i)
      if (owner && m_of[i] < dm) red[(wave * MP + m_of[i]) * kRowsWave + r] = acc[i];
  }
  if (kw > 1 || d.offset_mode != 0) __syncthreads();
  const bool lead = kp == 0;  // the tile's first wavefront finishes its rows
  if (lead && kw > 1) {
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
      if (owner && m_of[i] < dm) {
        float v = red[((tile * kw) * MP + m_of[i]) * kRowsWave + r];
        for (int pp = 1; pp < kw; ++pp) v += red[((tile * kw + pp) * MP + m_of[i]) * kRowsWave + r];
        acc[i] = v;
      }
    }
  }
  // ---- offsets over the item's range
  if (lead && d.offset_mode != 0) {
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
  if (RBLK > 0 && tid == 0) rot_release(f, wg, rot_mine);
  // ---- output
  const bool writer = lead && owner && row_ok;
  if (d.splits > 1) {
    if (writer) {
#pragma unroll
      for (int i = 0; i < NACC; ++i)
        if (m_of[i] < dm) part_store(d.partial + ((size_t)split * dm + m_of[i]) * d.n + row, acc[i]);
    }
    // with a counter, the row block's last part adds the parts in order
    if (d.ctr == nullptr || !last_part(d.ctr + rb, d.splits) || !writer) return;
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
      if (m_of[i] < dm) {
        float v = 0.f;
        for (int sp = 0; sp < d.splits; ++sp) v += part_load(d.partial + ((size_t)sp * dm + m_of[i]) * d.n + row);
        acc[i] = v;
      }
    }
  }
  if (!writer) return;
#pragma unroll
  for (int i = 0; i < NACC; ++i) {
    const int m = m_of[i];
    if (m < dm) {
      if (d.y_f32)
        reinterpret_cast<float*>(d.y)[(size_t)m * d.n + row] = acc[i];
      else
        reinterpret_cast<_Float16*>(d.y)[(size_t)m * d.n + row] = (_Float16)acc[i];
    }
  }
}

template <int G, int MP>
__global__ __launch_bounds__(kWave * kWaves) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_eu<G, MP>(), 8)))
void gemv_mfma_kernel(const GemvDesc* __restrict__ descs, const WgRec* __restrict__ recs, int ndesc, GemvDesc one) {
  RotFold none;
  none.shares = 0;
  mfma_body<G, MP, 0>(descs, recs, ndesc, one, none);
}

template <int G, int MP, int RBLK>
__global__ __launch_bounds__(kWave * kWaves) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_eu<G, MP>(), 8)))
void gemv_mfma_rot_kernel(const GemvDesc* __restrict__ descs, const WgRec* __restrict__ recs, int ndesc, RotFold f) {
  GemvDesc none;
  none.tile_begin = 0;
  mfma_body<G, MP, RBLK>(descs, recs, ndesc, none, f);
}

// Dynamic LDS of a launch (the layout the kernel computes, at its largest).
template <int G, int MP>
size_t mfma_lds_bytes(int max_krp, bool offsets) {
  const int ngr = max_krp / G;
  size_t lds = kZeroBytes + (size_t)MP * max_krp * 2 + ((size_t)kGemvRows * ngr * 2 + 32 + 15) / 16 * 16 +
               (size_t)kWaves * res_wave_bytes<MP>() + res_stage_bytes<G>() + (size_t)kWaves * MP * kRowsWave * 4;
  if (offsets) lds += (size_t)MP * (max_krp / G) * 4;
  return lds + 16;  // + the K-part arrival flag (static LDS)
}

template <int G, int MP>
hipError_t launch_mfma(const GemvDesc* descs, const WgRec* recs, int ndesc, const GemvDesc& one, int items, int max_krp,
                       bool offsets, hipStream_t s) {
  const size_t lds = mfma_lds_bytes<G, MP>(max_krp, offsets);
  hipLaunchKernelGGL((gemv_mfma_kernel<G, MP>), dim3(items), dim3(kWave * kWaves), lds, s, descs, recs, ndesc, one);
  return hipGetLastError();
}

template <int G, int MP>
hipError_t launch_mfma_rot(const GemvDesc* descs, const WgRec* recs, int ndesc, int items, int max_krp, bool offsets,
                           const RotFold& f, hipStream_t s) {
  const size_t lds = mfma_lds_bytes<G, MP>(max_krp, offsets);
  const dim3 grid((unsigned)(f.shares + items));
  if (f.block == 128)
    hipLaunchKernelGGL((gemv_mfma_rot_kernel<G, MP, 128>), grid, dim3(kWave * kWaves), lds, s, descs, recs, ndesc, f);
  else
    hipLaunchKernelGGL((gemv_mfma_rot_kernel<G, MP, 64>), grid, dim3(kWave * kWaves), lds, s, descs, recs, ndesc, f);
  return hipGetLastError();
}

template <int G>
hipError_t launch_mfma_g(int mp, const GemvDesc* descs, const WgRec* recs, int ndesc, const GemvDesc& one, int items,
                         int max_krp, bool offsets, hipStream_t s) {
  switch (mp) {
    case 1: return launch_mfma<G, 1>(descs, recs, ndesc, one, items, max_krp, offsets, s);
    case 2: return launch_mfma<G, 2>(descs, recs, ndesc, one, items, max_krp, offsets, s);
    case 4: return launch_mfma<G, 4>(descs, recs, ndesc, one, items, max_krp, offsets, s);
    case 8:
      if (G == 128) return launch_mfma<128, 8>(descs, recs, ndesc, one, items, max_krp, offsets, s);
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

__global__ void tile_bounds_kernel(const GemvDesc* ranges, WgRec* recs, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  WgRec* rec = recs + i;
  const GemvDesc* d = ranges + (rec->ri >> 20);
  const int item = (int)(rec->ri & 0xFFFFFu);
  const int row0 = d->row_base + (item % d->row_blocks) * kRowsWave * (kWaves / d->kwaves);
  if (d->pidx) {  // the item's K part in the index per K part
    const uint32_t* base = d->prowptr + (size_t)(item / d->row_blocks) * d->n;
    for (int t = 0; t < 5; ++t) rec->te[t] = base[min(row0 + kRowsWave * t, d->n)];
    return;
  }
  if (!d->gidx[0]) return;
  for (int t = 0; t < 5; ++t) rec->te[t] = d->rowptr[0][min(row0 + kRowsWave * t, d->n)];
}

// Index per K part: one thread per (part, row).  Residual planes are at
// most two; their masks, row pointers, blocks and scales come by value.
struct PartPlanes {
  const uint32_t* mask[2];
  const uint32_t* rowptr[2];
  const uint8_t* blocks[2];
  const uint16_t* rscale[2];
};

// The entries of (part s, row r) over planes p < nres, in plane then group
// order: group g of the part's range [ga, gb) with its mask bit set.
__device__ __forceinline__ uint32_t part_row_count(const PartPlanes& pp, int p, int r, int mwords, int ga, int gb) {
  const uint32_t* mrow = (p == 0 ? pp.mask[0] : pp.mask[1]) + (size_t)r * mwords;
  uint32_t c = 0;
  for (int w = ga >> 5; w <= (gb - 1) >> 5; ++w) c += __popc(mrow[w] & range_bits(ga - (w << 5), gb - (w << 5)));
  return c;
}

__global__ void part_count_kernel(PartPlanes pp, int nres, int n, int ng, int mwords, int parts, int gps,
                                  uint32_t* __restrict__ prowptr) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i == 0) prowptr[0] = 0u;
  if (i >= parts * n) return;
  const int s = i / n, r = i % n, ga = s * gps, gb = min(ng, ga + gps);
  uint32_t c = 0;
  for (int p = 0; p < nres; ++p) c += part_row_count(pp, p, r, mwords, ga, gb);
  prowptr[1 + i] = c;  // scanned in place next
}

template <int G>
__global__ void part_fill_kernel(PartPlanes pp, int nres, int n, int ng, int mwords, int gps,
                                 const uint32_t* __restrict__ prowptr, int parts, uint8_t* __restrict__ pblocks,
                                 uint32_t* __restrict__ pidx) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= parts * n) return;
  const int s = i / n, r = i % n, ga = s * gps, gb = min(ng, ga + gps);
  uint32_t e = prowptr[i];
  for (int p = 0; p < nres; ++p) {
    const uint32_t* mrow = (p == 0 ? pp.mask[0] : pp.mask[1]) + (size_t)r * mwords;
    const uint8_t* blocks = p == 0 ? pp.blocks[0] : pp.blocks[1];
    const uint16_t* rscale = p == 0 ? pp.rscale[0] : pp.rscale[1];
    // the row's entry number of group g: its row pointer plus the set bits before g
    uint32_t eo = (p == 0 ? pp.rowptr[0] : pp.rowptr[1])[r];
    for (int w = 0; w < (ga >> 5); ++w) eo += __popc(mrow[w]);
    if (ga & 31) eo += __popc(mrow[ga >> 5] & ((1u << (ga & 31)) - 1u));
    for (int w = ga >> 5; w <= (gb - 1) >> 5; ++w) {
      uint32_t bits = mrow[w] & range_bits(ga - (w << 5), gb - (w << 5));
      while (bits) {
        const int g = (w << 5) + __builtin_ctz(bits);
        bits &= bits - 1u;
        const uint4* src = reinterpret_cast<const uint4*>(blocks + (size_t)eo * (G / 4));
        uint4* dst = reinterpret_cast<uint4*>(pblocks + (size_t)e * (G / 4));
        for (int c = 0; c < G / 64; ++c) dst[c] = src[c];
        pidx[e] = (uint32_t)(g - ga) | ((uint32_t)rscale[eo] << 16);
        ++eo;
        ++e;
      }
    }
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

hipError_t launch_part_index(const uint32_t* const* mask, const uint32_t* const* rowptr, const uint8_t* const* blocks,
                             const uint16_t* const* rscale, int nres, int n, int ng, int mwords, int group, int parts,
                             int gps, uint32_t* prowptr, uint8_t* pblocks, uint32_t* pidx, hipStream_t s) {
  if (n <= 0 || parts <= 0 || nres < 1 || nres > 2 || gps <= 0) return hipErrorInvalidValue;
  PartPlanes pp;
  for (int p = 0; p < 2; ++p) {
    const int q = p < nres ? p : 0;
    pp.mask[p] = mask[q];
    pp.rowptr[p] = rowptr[q];
    pp.blocks[p] = blocks[q];
    pp.rscale[p] = rscale[q];
  }
  const int total = parts * n;
  const dim3 grid((unsigned)((total + 255) / 256));
  hipLaunchKernelGGL(part_count_kernel, grid, dim3(256), 0, s, pp, nres, n, ng, mwords, parts, gps, prowptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_rowptr_scan(prowptr, total, s);
  if (e != hipSuccess) return e;
  if (group == 128)
    hipLaunchKernelGGL(part_fill_kernel<128>, grid, dim3(256), 0, s, pp, nres, n, ng, mwords, gps, prowptr, parts,
                       pblocks, pidx);
  else if (group == 64)
    hipLaunchKernelGGL(part_fill_kernel<64>, grid, dim3(256), 0, s, pp, nres, n, ng, mwords, gps, prowptr, parts,
                       pblocks, pidx);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_tile_bounds(const GemvDesc* ranges, WgRec* recs, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(tile_bounds_kernel, dim3((count + 255) / 256), dim3(256), 0, s, ranges, recs, count);
  return hipGetLastError();
}

int gemv_mfma_max_rows(int group) { return group == 128 ? 8 : 4; }

int gemv_mfma_wgs_per_cu(int group, int mp, int max_krp, bool offsets) {
  // 160 KB of LDS per CU; one wavefront of a workgroup per SIMD
  size_t lds = 0;
  int wpe = 3;
  if (group == 128) {
    lds = mp == 1 ? mfma_lds_bytes<128, 1>(max_krp, offsets) : mp == 2 ? mfma_lds_bytes<128, 2>(max_krp, offsets)
        : mp == 4 ? mfma_lds_bytes<128, 4>(max_krp, offsets) : mfma_lds_bytes<128, 8>(max_krp, offsets);
    wpe = mp == 8 ? mfma_waves_per_eu<128, 8>() : 3;
  } else {
    lds = mp == 1 ? mfma_lds_bytes<64, 1>(max_krp, offsets) : mp == 2 ? mfma_lds_bytes<64, 2>(max_krp, offsets)
        : mfma_lds_bytes<64, 4>(max_krp, offsets);
    wpe = mp == 4 ? mfma_waves_per_eu<64, 4>() : 3;
  }
  const int by_lds = lds ? (int)((160u * 1024u) / lds) : wpe;
  return std::max(1, std::min(by_lds, wpe));
}

int gemv_mfma_max_range(int mp) { return std::min(16384 / mp, kMaxBlocks * kBlockTrits * kWaves); }

hipError_t launch_gemv_mfma(int group, int mp, const GemvDesc* descs, const WgRec* recs, int ndesc, const GemvDesc& one,
                            int total_items, int max_krp, bool offsets, hipStream_t s) {
  if (total_items <= 0) return hipSuccess;
  if (ndesc > 0 && !recs) return hipErrorInvalidValue;
  if (group == 64) return launch_mfma_g<64>(mp, descs, recs, ndesc, one, total_items, max_krp, offsets, s);
  if (group == 128) return launch_mfma_g<128>(mp, descs, recs, ndesc, one, total_items, max_krp, offsets, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_mfma_rot(int group, int mp, const GemvDesc* descs, const WgRec* recs, int ndesc,
                                int total_items, int max_krp, bool offsets, const RotFold& f, hipStream_t s) {
  if (total_items <= 0) return hipSuccess;
  if (ndesc <= 0 || !recs || !f.sync || f.shares < 0 || f.a.m > mp || !(f.block == 64 || f.block == 128))
    return hipErrorInvalidValue;
  if (f.shares == 0) {
    GemvDesc unused;
    std::memset(&unused, 0, sizeof(unused));
    return launch_gemv_mfma(group, mp, descs, recs, ndesc, unused, total_items, max_krp, offsets, s);
  }
  switch (group * 16 + mp) {
    case 128 * 16 + 1: return launch_mfma_rot<128, 1>(descs, recs, ndesc, total_items, max_krp, offsets, f, s);
    case 128 * 16 + 2: return launch_mfma_rot<128, 2>(descs, recs, ndesc, total_items, max_krp, offsets, f, s);
    case 128 * 16 + 4: return launch_mfma_rot<128, 4>(descs, recs, ndesc, total_items, max_krp, offsets, f, s);
    case 128 * 16 + 8: return launch_mfma_rot<128, 8>(descs, recs, ndesc, total_items, max_krp, offsets, f, s);
    case 64 * 16 + 1: return launch_mfma_rot<64, 1>(descs, recs, ndesc, total_items, max_krp, offsets, f, s);
    case 64 * 16 + 2: return launch_mfma_rot<64, 2>(descs, recs, ndesc, total_items, max_krp, offsets, f, s);
    case 64 * 16 + 4: return launch_mfma_rot<64, 4>(descs, recs, ndesc, total_items, max_krp, offsets, f, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tern
