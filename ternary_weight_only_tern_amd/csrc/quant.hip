// Quantizer front-end: FP16 weights -> two trit planes, FP16 scales and
// per-group FP16 offsets, the inputs of tern_pack with per-group offsets.
//
// Method: E2M-ATQ, order-2 asymmetric residual ternarization ("Post-Training
// Ternarization of Qwen3-4B", arXiv 2609.01962v1 summary, §4.3): an offset
// plus two ternary planes with scales per group, then 15 refinement
// iterations with the ternary supports held fixed; the second plane only on
// salience-selected groups (§4.4; here a caller-supplied mask per (row,
// group)), groups of 128 (§4.5).  The pages leave the initial threshold and
// the content of an iteration open; this kernel takes:
//   * initial supports by the ternary-weight-network threshold: with
//     r = w - mean(w), non-zero where |r| > 0.7 mean|r|, sign of r, first
//     scale mean|r| over the support; the second plane applies the same rule
//     to r - alpha t0 (masked groups only);
//   * an iteration = the least-squares fit of (mu, s0, s1) over the basis
//     (1, t0, t1) (normal equations by Cramer's rule; a singular system drops
//     s1, then s0), then the error-minimizing sign of every non-zero trit
//     given the fit (plane 0, then plane 1 with the new plane 0); a last fit
//     after the iterations gives the stored values.
//
// Decisions depend on floating-point sums, so every quantity is computed in
// FP32 with one fixed order: a group sum pairs element i with i + G/2, then
// halves again, and no multiply-add is contracted.  Results are therefore
// reproducible bit for bit.  Sixteen lanes share a group: lane l holds
// elements l + 16 j, so the first halvings (i + 64, i + 32, i + 16) are adds
// inside the lane and the last four are xor shuffles 8, 4, 2, 1, which give
// the group's sixteen lanes the same total bit for bit; a wavefront
// quantizes four groups.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "internal.h"

#pragma clang fp contract(off)

namespace tern {
namespace {

constexpr int kWave = 64;
constexpr int kLanes = 16;  // lanes per group

// Sum over the group's E * 16 elements in the fixed halving order.
template <int E>
__device__ __forceinline__ float group_sum(const float (&v)[E]) {
  float t[E];
#pragma unroll
  for (int j = 0; j < E; ++j) t[j] = v[j];
#pragma unroll
  for (int h = E / 2; h >= 1; h /= 2)
#pragma unroll
    for (int j = 0; j < h; ++j) t[j] = t[j] + t[j + h];
  float x = t[0];
#pragma unroll
  for (int o = kLanes / 2; o > 0; o >>= 1) x = x + __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ int8_t sign_of(float x) { return x < 0.f ? (int8_t)-1 : (int8_t)1; }

struct Fit {
  float mu, a, b;
};

// Least-squares (mu, a, b) of w over (1, t0, t1); sw, n0, n1: sum of w and
// the support sizes (fixed), g: the group size.
template <int E>
__device__ __forceinline__ Fit fit(const float (&w)[E], const int8_t (&t0)[E], const int8_t (&t1)[E], bool masked,
                                   float sw, float n0, float n1, float g) {
  float f0[E], f1[E], f01[E], w0[E], w1[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    f0[e] = (float)t0[e];
    f1[e] = (float)t1[e];
    f01[e] = f0[e] * f1[e];
    w0[e] = w[e] * f0[e];
    w1[e] = w[e] * f1[e];
  }
  const float p0 = group_sum<E>(f0), p1 = group_sum<E>(f1), c01 = group_sum<E>(f01);
  const float sw0 = group_sum<E>(w0), sw1 = group_sum<E>(w1);
  Fit f;
  const float m00 = n0 * n1 - c01 * c01;
  const float m01 = p1 * c01 - p0 * n1;
  const float m02 = p0 * c01 - p1 * n0;
  const float det3 = (g * m00 + p0 * m01) + p1 * m02;
  if (masked && n1 > 0.f && det3 != 0.f) {
    f.mu = ((sw * m00 + sw0 * m01) + sw1 * m02) / det3;
    const float da = (g * (sw0 * n1 - c01 * sw1) - sw * (p0 * n1 - c01 * p1)) + p1 * (p0 * sw1 - sw0 * p1);
    const float db = (g * (n0 * sw1 - sw0 * c01) - p0 * (p0 * sw1 - sw0 * p1)) + sw * (p0 * c01 - n0 * p1);
    f.a = da / det3;
    f.b = db / det3;
    return f;
  }
  const float det2 = g * n0 - p0 * p0;
  if (n0 > 0.f && det2 != 0.f) {
    f.mu = (sw * n0 - p0 * sw0) / det2;
    f.a = (g * sw0 - p0 * sw) / det2;
  } else {
    f.mu = sw / g;
    f.a = 0.f;
  }
  f.b = 0.f;
  return f;
}

// Sixteen lanes per (row, group): groups grp = row * ng + g, four per
// wavefront.
template <int G>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ wt, int n, int k,
                                                       const uint32_t* __restrict__ mask, int mwords, int iters,
                                                       int8_t* __restrict__ trits, uint16_t* __restrict__ scales,
                                                       uint16_t* __restrict__ offset) {
  constexpr int E = G / kLanes;
  const int ng = k / G;
  const long total = (long)n * ng;
  const long gq = (long)blockIdx.x * (256 / kLanes) + threadIdx.x / kLanes;
  const bool live = gq < total;  // the last wavefront may hold fewer groups
  const long grp = live ? gq : total - 1;
  const int lane = threadIdx.x % kLanes;
  const int row = (int)(grp / ng), g = (int)(grp % ng);
  const size_t base = (size_t)row * k + (size_t)g * G;
  float w[E];
#pragma unroll
  for (int e = 0; e < E; ++e) w[e] = (float)__builtin_bit_cast(_Float16, wt[base + lane + kLanes * e]);
  const bool masked = mask != nullptr && ((mask[(size_t)row * mwords + g / 32] >> (g % 32)) & 1u);
  const float inv = 1.0f / (float)G, gf = (float)G;

  // initial supports
  const float sw = group_sum<E>(w);
  const float mu0 = sw * inv;
  float r[E], a[E], on[E], aon[E];
  int8_t t0[E], t1[E];
  bool on0[E], on1[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    r[e] = w[e] - mu0;
    a[e] = fabsf(r[e]);
  }
  const float thr = (group_sum<E>(a) * inv) * 0.7f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    on0[e] = a[e] > thr;
    t0[e] = on0[e] ? sign_of(r[e]) : (int8_t)0;
    on[e] = on0[e] ? 1.f : 0.f;
    aon[e] = on0[e] ? a[e] : 0.f;
  }
  const float n0 = group_sum<E>(on);
  const float s_on = group_sum<E>(aon);
  const float alpha = n0 > 0.f ? s_on / fmaxf(n0, 1.f) : 0.f;
  float a2[E], r2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    r2[e] = r[e] - alpha * (float)t0[e];
    a2[e] = fabsf(r2[e]);
  }
  const float thr2 = (group_sum<E>(a2) * inv) * 0.7f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    on1[e] = masked && a2[e] > thr2;
    t1[e] = on1[e] ? sign_of(r2[e]) : (int8_t)0;
    on[e] = on1[e] ? 1.f : 0.f;
  }
  const float n1 = group_sum<E>(on);

  // refinement, supports fixed
  for (int it = 0; it < iters; ++it) {
    const Fit f = fit<E>(w, t0, t1, masked, sw, n0, n1, gf);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float e0 = (w[e] - f.mu) - f.b * (float)t1[e];
      t0[e] = on0[e] ? sign_of(f.a * e0) : (int8_t)0;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float e1 = (w[e] - f.mu) - f.a * (float)t0[e];
      t1[e] = on1[e] ? sign_of(f.b * e1) : (int8_t)0;
    }
  }
  const Fit f = fit<E>(w, t0, t1, masked, sw, n0, n1, gf);

  if (!live) return;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    trits[base + lane + kLanes * e] = t0[e];
    trits[(size_t)n * k + base + lane + kLanes * e] = t1[e];
  }
  if (lane == 0) {
    const size_t sg = (size_t)row * ng + g;
    scales[sg] = __builtin_bit_cast(uint16_t, (_Float16)f.a);
    scales[(size_t)n * ng + sg] = __builtin_bit_cast(uint16_t, (_Float16)f.b);
    offset[sg] = __builtin_bit_cast(uint16_t, (_Float16)f.mu);
  }
}

}  // namespace

hipError_t launch_quantize(const uint16_t* w, int n, int k, int group, const uint32_t* mask, int mwords, int iters,
                           int8_t* trits, uint16_t* scales, uint16_t* offset, hipStream_t s) {
  const long groups = (long)n * (k / group);
  if (groups <= 0) return hipSuccess;
  const dim3 grid((unsigned)((groups + 15) / 16));
  if (group == 128)
    hipLaunchKernelGGL((quantize_kernel<128>), grid, dim3(256), 0, s, w, n, k, mask, mwords, iters, trits, scales,
                       offset);
  else
    hipLaunchKernelGGL((quantize_kernel<64>), grid, dim3(256), 0, s, w, n, k, mask, mwords, iters, trits, scales,
                       offset);
  return hipGetLastError();
}

}  // namespace tern
