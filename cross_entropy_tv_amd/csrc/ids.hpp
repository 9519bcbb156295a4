// Work-item and grid indices for the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace lx {

// Work-item and grid indices read straight from the hardware and the dispatch
// packet.  The kernels are compiled with IEEE mode off, the device library's
// index functions with it on, and the compiler does not inline a function
// built for another floating-point mode: threadIdx / blockIdx / blockDim /
// gridDim would each become a real call, with the calling convention's
// register traffic around it.
__device__ __forceinline__ int tid_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ unsigned bid_x() { return __builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ unsigned bdim_x() { return __builtin_amdgcn_workgroup_size_x(); }
// The number of workgroups is the first implicit kernel argument (code object
// v5 layout), which sits with the explicit ones in the kernel-argument
// segment.  The dispatch packet also holds the grid size, but the packet lives
// in the queue's ring buffer: reading it at every workgroup's start measurably
// slowed kernels made of many short workgroups.
__device__ __forceinline__ unsigned nblocks_x() {
  return *(const unsigned*)__builtin_amdgcn_implicitarg_ptr();
}

}  // namespace lx
