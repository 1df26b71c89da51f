// Activation-side rotation: xr = R x with R block diagonal (B x B blocks,
// B = 64 or 128), applied before the packed product.  "Post-Training
// Ternarization of Qwen3-4B" (arXiv 2609.01962v1 summary) §4.2: the weights
// live in a rotated basis (KOTMS, structured orthogonal matrices) and
// inference applies the matching rotation to the activations first; the
// pages do not give the structure, so R is any caller-supplied
// block-diagonal matrix aligned with the weight groups.
//
// One workgroup of 256 threads per (block, chunk of up to kRows activation
// rows): R_b is copied to LDS with contiguous 16-byte loads (its rows padded
// by one 4-byte word, so that the threads' row reads below fall in distinct
// banks) and the block's activations with contiguous 4-byte loads (x and out
// need only 4-byte alignment); thread t computes output row
// t % B of activation rows t / B, t / B + 256 / B, ... with v_dot2_f32_f16
// over the FP16 pairs of its row (FP16 products are exact in FP32);
// outputs are FP16 (round to nearest even).  A workgroup reads its
// activations before writing any output, and no other workgroup touches
// them, so out may equal x.  Up to kMaxRotations inputs (a layer's q/k/v and
// gate/up input, attention output and MLP intermediate, say) share one
// launch: their pointers travel in the kernel arguments and workgroup j
// belongs to the input whose block range holds j.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "internal.h"

namespace tern {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kRows = 16;  // activation rows per workgroup

template <int B>
__global__ __launch_bounds__(256) void rotate_kernel(RotBatch a) {
  constexpr int P = B / 2 + 1;  // padded row pitch of R in LDS (FP16 pairs)
  __shared__ uint32_t rs[B * P];
  __shared__ uint32_t xs[kRows * B / 2];  // [row][B/2] FP16 pairs
  int in = 0;
  while (in + 1 < a.count && (int)blockIdx.x >= a.begin[in + 1]) ++in;
  const uint16_t* __restrict__ R = a.R[in];
  const uint16_t* x = a.x[in];
  uint16_t* out = a.out[in];
  const int k = a.k[in], m = a.m;
  const int b = (int)blockIdx.x - a.begin[in];
  const int m0 = blockIdx.y * kRows;
  const int rows = min(kRows, m - m0);
  const int t = threadIdx.x;
  // R_b: B rows of B / 8 16-byte chunks, every chunk of the thread requested
  // before any is stored
  constexpr int NC = B * (B / 8) / 256;
  const u4_t* rg = reinterpret_cast<const u4_t*>(R + (size_t)b * B * B);
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
  for (int e = t; e < rows * (B / 2); e += 256) {
    const int r = e / (B / 2), j = e % (B / 2);
    xs[e] = reinterpret_cast<const uint32_t*>(x + (size_t)(m0 + r) * k + (size_t)b * B)[j];
  }
  __syncthreads();
  const int i = t % B;
  const uint32_t* ri = rs + i * P;
  for (int r = t / B; r < rows; r += 256 / B) {
    const uint32_t* xr = xs + r * (B / 2);
    float acc = 0.f;
#pragma unroll 16
    for (int j = 0; j < B / 2; ++j)
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, ri[j]), __builtin_bit_cast(h2_t, xr[j]), acc, false);
    out[(size_t)(m0 + r) * k + (size_t)b * B + i] = __builtin_bit_cast(uint16_t, (_Float16)acc);
  }
}

}  // namespace

hipError_t launch_rotate(const RotBatch& a, int block, hipStream_t s) {
  const int blocks = a.begin[a.count];
  if (a.m <= 0 || blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks, (unsigned)((a.m + kRows - 1) / kRows));
  if (block == 128)
    hipLaunchKernelGGL((rotate_kernel<128>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((rotate_kernel<64>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tern
