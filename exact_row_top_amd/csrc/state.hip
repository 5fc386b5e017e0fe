// state.hip -- device-side state the library keeps per GPU, and the kernels
// that read and reset it.
//
//  * timeout_count: the split tier's row barriers are bounded waits (its
//    workgroups rely on being resident together); a wait that gives up adds
//    one here and lets its workgroup run on, so that every wave still exits.
//    The results of such a call are undefined.  topk_status hands the count to
//    the caller in stream order and resets it.
//  * scratch: the split tier's workspace for topk_decode_noalloc, for callers
//    that cannot allocate (graph capture, serving loops that forbid
//    hipMalloc).  It holds the same layout a caller workspace does, rests at
//    zero between calls, and is shared by every such call on the GPU: calls
//    that overlap on one GPU race.
//
// File-scope __device__ variables exist once per GPU the library runs on;
// host code reaches each GPU's copy through the address hipGetSymbolAddress
// returns with that GPU current (the host-side name is only a stand-in).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gvr_common.h"

namespace ert {

static __device__ uint32_t timeout_count;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Address of this GPU's timeout count (the current device).  Returns a HIP
// status.
hipError_t state_timeout_address(uint32_t** out) {
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(timeout_count));
  *out = static_cast<uint32_t*>(p);
  return e;
}

// Address of this GPU's scratch array (the current device); a HIP status.
hipError_t state_scratch_address(void** out) {
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  *out = p;
  return e;
}

// Zero n 16-byte words (graph-safe: a kernel, not a memset node).
__global__ void __launch_bounds__(256) fill_zero_kernel(uint4* p, size_t n) {
  const uint4 z{0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = z;
}

// Every workgroup reads the count; the first thread of the grid hands it to
// the caller.  With a non-zero count, the workgroups zero the library-owned
// buffers whose split-tier slots a timed-out call may have left away from
// their resting state, each its grid-stride share of 16-byte words.
__global__ void __launch_bounds__(256)
    status_read_kernel(const uint32_t* count, int32_t* out, uint4* buf0, size_t n0, uint4* buf1,
                       size_t n1) {
  const uint32_t c = __hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t step = (size_t)gridDim.x * blockDim.x;
  if (i0 == 0) *out = (int32_t)(c > 0x7FFFFFFFu ? 0x7FFFFFFFu : c);
  if (c == 0u) return;
  const uint4 z{0u, 0u, 0u, 0u};
  for (size_t i = i0; i < n0; i += step) buf0[i] = z;
  for (size_t i = i0; i < n1; i += step) buf1[i] = z;
}

// Runs after status_read_kernel on the same stream: back to zero.
__global__ void status_reset_kernel(uint32_t* count) {
  if (threadIdx.x == 0 && blockIdx.x == 0)
    __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

const void* fill_zero_kernel_ptr() { return reinterpret_cast<const void*>(&fill_zero_kernel); }
const void* status_read_kernel_ptr() { return reinterpret_cast<const void*>(&status_read_kernel); }
const void* status_reset_kernel_ptr() { return reinterpret_cast<const void*>(&status_reset_kernel); }

}  // namespace ert
