// Packing and unpacking of trit planes (the lossless serialisation step:
// "Post-Training Ternarization of Qwen3-4B", §9.1 and §15; arXiv 2609.09240,
// packing paragraph).  Cold path: one thread per output unit, validation
// results are OR-ed into a device flag that the host reads back.
#include "internal.h"

namespace tern {
namespace {

constexpr int kThreads = 256;

__device__ inline void raise_flag(uint32_t* flag, uint32_t bit) { atomicOr(flag, bit); }

// Bit position of the trit at offset o (0..15) inside its 32-bit word: even
// offsets fill the low half-word, odd offsets the high half-word.
__device__ __forceinline__ int bitpos(int o) { return ((o & 1) << 4) | ((o >> 1) << 1); }

// ---------------------------------------------------------------- 2-bit plane 0
__global__ void pack_2bit_kernel(const int8_t* __restrict__ trits, int n, int k,
                                 uint8_t* __restrict__ out, uint32_t* flag) {
  const int words_per_row = k >> 4;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)n * words_per_row) return;
  const size_t row = idx / words_per_row;
  const int w = (int)(idx % words_per_row);
  const uint4 v = *reinterpret_cast<const uint4*>(trits + row * k + (size_t)w * 16);
  const uint32_t lanes[4] = {v.x, v.y, v.z, v.w};
  uint32_t word = 0;
  bool bad = false;
#pragma unroll
  for (int o = 0; o < 16; ++o) {
    const int t = (int)(int8_t)((lanes[o >> 2] >> ((o & 3) * 8)) & 0xFF);
    bad |= (t < -1) | (t > 1);
    word |= (uint32_t)(t & 3) << bitpos(o);
  }
  if (bad) raise_flag(flag, kFlagBadTrit);
  reinterpret_cast<uint32_t*>(out + row * (size_t)(k >> 2))[w] = word;
}

__global__ void unpack_2bit_kernel(const uint8_t* __restrict__ in, int n, int k,
                                   int8_t* __restrict__ trits, uint32_t* flag) {
  const int words_per_row = k >> 4;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)n * words_per_row) return;
  const size_t row = idx / words_per_row;
  const int w = (int)(idx % words_per_row);
  const uint32_t word = reinterpret_cast<const uint32_t*>(in + row * (size_t)(k >> 2))[w];
  uint32_t lanes[4] = {0, 0, 0, 0};
  bool bad = false;
#pragma unroll
  for (int o = 0; o < 16; ++o) {
    const uint32_t code = (word >> bitpos(o)) & 3u;
    bad |= code == 2u;
    const uint32_t t = code == 3u ? 0xFFu : code;  // int8 -1 / 0 / 1
    lanes[o >> 2] |= t << ((o & 3) * 8);
  }
  if (bad) raise_flag(flag, kFlagBadCode);
  *reinterpret_cast<uint4*>(trits + row * k + (size_t)w * 16) =
      make_uint4(lanes[0], lanes[1], lanes[2], lanes[3]);
}

// ---------------------------------------------------------------- base-3 plane 0
__global__ void pack_b3_kernel(const int8_t* __restrict__ trits, int n, int k, int group,
                               int stride, uint8_t* __restrict__ out, uint32_t* flag) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)n * stride) return;
  const size_t row = idx / stride;
  const int j = (int)(idx % stride);
  const int gb = (group + 4) / 5;
  const int ng = k / group;
  uint32_t v = 0;
  if (j < ng * gb) {
    const int g = j / gb, jj = j % gb;
    const int8_t* src = trits + row * k + (size_t)g * group;
    bool bad = false;
    uint32_t p3 = 1;
    for (int i = 0; i < 5; ++i) {
      const int pos = 5 * jj + i;
      int t = 0;
      if (pos < group) {
        t = src[pos];
        bad |= (t < -1) | (t > 1);
      }
      v += (uint32_t)(t + 1) * p3;
      p3 *= 3;
    }
    if (bad) {
      raise_flag(flag, kFlagBadTrit);
      v = 0;
    }
  }
  out[idx] = (uint8_t)v;
}

__global__ void unpack_b3_kernel(const uint8_t* __restrict__ in, int n, int k, int group,
                                 int stride, int8_t* __restrict__ trits, uint32_t* flag) {
  const int gb = (group + 4) / 5;
  const int ng = k / group;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)n * ng * gb) return;
  const size_t row = idx / ((size_t)ng * gb);
  const int rem = (int)(idx % ((size_t)ng * gb));
  const int g = rem / gb, jj = rem % gb;
  uint32_t v = in[row * stride + (size_t)g * gb + jj];
  bool bad = v > 242u;
  int8_t* dst = trits + row * k + (size_t)g * group;
  for (int i = 0; i < 5; ++i) {
    const int d = (int)(v % 3u);
    v /= 3u;
    const int pos = 5 * jj + i;
    if (pos < group)
      dst[pos] = (int8_t)(d - 1);
    else
      bad |= d != 1;
  }
  if (bad) raise_flag(flag, kFlagBadCode);
}

// ---------------------------------------------------------------- residual planes
__device__ __forceinline__ uint32_t mask_bit(const uint32_t* row_mask, int g) {
  return (row_mask[g >> 5] >> (g & 31)) & 1u;
}

// Number of set bits strictly below group g in one row's bitmap.
__device__ __forceinline__ uint32_t rank_below(const uint32_t* row_mask, int g) {
  uint32_t c = 0;
  for (int w = 0; w < (g >> 5); ++w) c += __popc(row_mask[w]);
  const uint32_t low = (g & 31) ? (row_mask[g >> 5] & ((1u << (g & 31)) - 1u)) : 0u;
  return c + __popc(low);
}

__global__ void mask_counts_kernel(const uint32_t* __restrict__ mask, int n, int ng, int mwords,
                                   uint32_t* __restrict__ rowptr, uint32_t* flag) {
  const int row = blockIdx.x * kThreads + threadIdx.x;
  if (row == 0) rowptr[0] = 0;
  if (row >= n) return;
  const uint32_t* m = mask + (size_t)row * mwords;
  uint32_t c = 0;
  for (int w = 0; w < mwords; ++w) c += __popc(m[w]);
  const int tail = ng & 31;
  if (tail && (m[mwords - 1] >> tail)) raise_flag(flag, kFlagMaskBits);
  rowptr[row + 1] = c;
}

// Inclusive scan of rowptr[1..n] with one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void rowptr_scan_kernel(uint32_t* rowptr, int n) {
  __shared__ uint32_t buf[1024];
  __shared__ uint32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + (int)threadIdx.x;
    uint32_t v = i < n ? rowptr[1 + i] : 0u;
    buf[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const uint32_t add = threadIdx.x >= (unsigned)off ? buf[threadIdx.x - off] : 0u;
      __syncthreads();
      buf[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < n) rowptr[1 + i] = buf[threadIdx.x] + carry;
    __syncthreads();
    if (threadIdx.x == 1023) carry += buf[1023];
    __syncthreads();
  }
}

__global__ void pack_residual_kernel(const int8_t* __restrict__ trits_p,
                                     const uint16_t* __restrict__ rscale_dense,
                                     const uint32_t* __restrict__ mask,
                                     const uint32_t* __restrict__ rowptr, int n, int k, int group,
                                     int mwords, uint8_t* __restrict__ blocks,
                                     uint16_t* __restrict__ rscale, uint32_t* flag) {
  const int ng = k / group;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)n * ng) return;
  const int row = (int)(idx / ng), g = (int)(idx % ng);
  const uint32_t* rm = mask + (size_t)row * mwords;
  const int8_t* src = trits_p + (size_t)row * k + (size_t)g * group;
  if (!mask_bit(rm, g)) {
    bool nz = false;
    for (int i = 0; i < group; i += 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + i);
      nz |= (v.x | v.y | v.z | v.w) != 0u;
    }
    if (nz) raise_flag(flag, kFlagOutsideMask);
    return;
  }
  const uint32_t b = rowptr[row] + rank_below(rm, g);
  uint32_t* dst = reinterpret_cast<uint32_t*>(blocks + (size_t)b * (group >> 2));
  bool bad = false;
  for (int w = 0; w < (group >> 4); ++w) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + w * 16);
    const uint32_t lanes[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0;
#pragma unroll
    for (int o = 0; o < 16; ++o) {
      const int t = (int)(int8_t)((lanes[o >> 2] >> ((o & 3) * 8)) & 0xFF);
      bad |= (t < -1) | (t > 1);
      word |= (uint32_t)(t & 3) << bitpos(o);
    }
    dst[w] = word;
  }
  if (bad) raise_flag(flag, kFlagBadTrit);
  rscale[b] = rscale_dense[(size_t)row * ng + g];
}

__global__ void unpack_residual_kernel(const uint8_t* __restrict__ blocks,
                                       const uint32_t* __restrict__ mask,
                                       const uint32_t* __restrict__ rowptr, int n, int k,
                                       int group, int mwords, int8_t* __restrict__ trits_p,
                                       uint32_t* flag) {
  const int ng = k / group;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)n * ng) return;
  const int row = (int)(idx / ng), g = (int)(idx % ng);
  const uint32_t* rm = mask + (size_t)row * mwords;
  int8_t* dst = trits_p + (size_t)row * k + (size_t)g * group;
  if (!mask_bit(rm, g)) {
    for (int i = 0; i < group; i += 16) *reinterpret_cast<uint4*>(dst + i) = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint32_t b = rowptr[row] + rank_below(rm, g);
  const uint32_t* src = reinterpret_cast<const uint32_t*>(blocks + (size_t)b * (group >> 2));
  bool bad = false;
  for (int w = 0; w < (group >> 4); ++w) {
    const uint32_t word = src[w];
    uint32_t lanes[4] = {0, 0, 0, 0};
#pragma unroll
    for (int o = 0; o < 16; ++o) {
      const uint32_t code = (word >> bitpos(o)) & 3u;
      bad |= code == 2u;
      lanes[o >> 2] |= (code == 3u ? 0xFFu : code) << ((o & 3) * 8);
    }
    *reinterpret_cast<uint4*>(dst + w * 16) = make_uint4(lanes[0], lanes[1], lanes[2], lanes[3]);
  }
  if (bad) raise_flag(flag, kFlagBadCode);
}

__global__ void compare_u32_kernel(const uint32_t* a, const uint32_t* b, int count, uint32_t bit,
                                   uint32_t* flag) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < count && a[i] != b[i]) raise_flag(flag, bit);
}

inline unsigned blocks_for(size_t work) { return (unsigned)((work + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_pack_plane0(int format, const int8_t* trits, int n, int k, int group, int stride,
                              uint8_t* plane0, uint32_t* flag, hipStream_t s) {
  if (format == 0) {
    const size_t work = (size_t)n * (k >> 4);
    if (work) hipLaunchKernelGGL(pack_2bit_kernel, dim3(blocks_for(work)), dim3(kThreads), 0, s, trits, n, k, plane0, flag);
  } else {
    const size_t work = (size_t)n * stride;
    if (work) hipLaunchKernelGGL(pack_b3_kernel, dim3(blocks_for(work)), dim3(kThreads), 0, s, trits, n, k, group, stride, plane0, flag);
  }
  return hipGetLastError();
}

hipError_t launch_unpack_plane0(int format, const uint8_t* plane0, int n, int k, int group,
                                int stride, int8_t* trits, uint32_t* flag, hipStream_t s) {
  if (format == 0) {
    const size_t work = (size_t)n * (k >> 4);
    if (work) hipLaunchKernelGGL(unpack_2bit_kernel, dim3(blocks_for(work)), dim3(kThreads), 0, s, plane0, n, k, trits, flag);
  } else {
    const size_t work = (size_t)n * (k / group) * ((group + 4) / 5);
    if (work) hipLaunchKernelGGL(unpack_b3_kernel, dim3(blocks_for(work)), dim3(kThreads), 0, s, plane0, n, k, group, stride, trits, flag);
  }
  return hipGetLastError();
}

hipError_t launch_mask_counts(const uint32_t* mask, int n, int ng, int mwords, uint32_t* rowptr,
                              uint32_t* flag, hipStream_t s) {
  hipLaunchKernelGGL(mask_counts_kernel, dim3(blocks_for((size_t)(n > 0 ? n : 1))), dim3(kThreads), 0, s,
                     mask, n, ng, mwords, rowptr, flag);
  return hipGetLastError();
}

hipError_t launch_rowptr_scan(uint32_t* rowptr, int n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(rowptr_scan_kernel, dim3(1), dim3(1024), 0, s, rowptr, n);
  return hipGetLastError();
}

hipError_t launch_pack_residual(const int8_t* trits_p, const uint16_t* rscale_dense,
                                const uint32_t* mask, const uint32_t* rowptr, int n, int k,
                                int group, int mwords, uint8_t* blocks, uint16_t* rscale,
                                uint32_t* flag, hipStream_t s) {
  const size_t work = (size_t)n * (k / group);
  if (work) hipLaunchKernelGGL(pack_residual_kernel, dim3(blocks_for(work)), dim3(kThreads), 0, s,
                               trits_p, rscale_dense, mask, rowptr, n, k, group, mwords, blocks, rscale, flag);
  return hipGetLastError();
}

hipError_t launch_unpack_residual(const uint8_t* blocks, const uint32_t* mask, const uint32_t* rowptr,
                                  int n, int k, int group, int mwords, int8_t* trits_p,
                                  uint32_t* flag, hipStream_t s) {
  const size_t work = (size_t)n * (k / group);
  if (work) hipLaunchKernelGGL(unpack_residual_kernel, dim3(blocks_for(work)), dim3(kThreads), 0, s,
                               blocks, mask, rowptr, n, k, group, mwords, trits_p, flag);
  return hipGetLastError();
}

hipError_t launch_compare_u32(const uint32_t* a, const uint32_t* b, int count, uint32_t bit,
                              uint32_t* flag, hipStream_t s) {
  if (count > 0) hipLaunchKernelGGL(compare_u32_kernel, dim3(blocks_for((size_t)count)), dim3(kThreads), 0, s,
                                    a, b, count, bit, flag);
  return hipGetLastError();
}

}  // namespace tern
