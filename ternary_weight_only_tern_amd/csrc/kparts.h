// K parts summed inside the decode launch.  The workgroups of one row block
// that cover different K parts each store their FP32 partial sums, then
// count themselves in at the block's arrival counter; the last to arrive
// adds the parts in part order (so the result does not depend on which
// workgroup is last) and writes y.  Nothing waits on another workgroup.
//
// Partials are written through to the device-coherent level (agent-scope
// stores, which bypass the per-XCD L2) and read back the same way, so no
// cache-wide writeback or invalidate is needed: a device-scope fence here
// writes back and invalidates the whole L2 of the XCD and costs more than
// the separate reduce launch it replaces.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tern {

// A partial sum for another workgroup of the launch.
__device__ __forceinline__ void part_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A partial sum written by another workgroup of the launch.
__device__ __forceinline__ float part_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every thread of the workgroup after its part_store()s.  Returns
// true in every thread of the row block's last workgroup (whose part_load()s
// then see every part); that workgroup also resets the counter to zero for
// the next launch.
__device__ __forceinline__ bool last_part(uint32_t* ctr, int splits) {
  __shared__ uint32_t last_flag;
  // this thread's stores are acknowledged by the coherent level (vmcnt(0))
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();  // ... for every thread of the workgroup
  if (threadIdx.x == 0) {
    const uint32_t before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = before + 1u == (uint32_t)splits;
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = last ? 1u : 0u;
  }
  __syncthreads();
  return last_flag != 0u;
}

// The same for a single wavefront that owns a whole work item (no workgroup
// barrier): true in every lane of the wavefront that adds the parts.
__device__ __forceinline__ bool last_part_wave(uint32_t* ctr, int splits, int lane) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // this wavefront's part stores are acknowledged
  uint32_t before = 0u;
  if (lane == 0) before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  before = __shfl(before, 0, 64);
  const bool last = before + 1u == (uint32_t)splits;
  if (last && lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

}  // namespace tern
