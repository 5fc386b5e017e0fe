// epilogue.hip -- optional output stage after the selection kernels:
//  * the values of the selected scores (a destination-passing values array;
//    short rows keep their identity indices and pad values with -FLT_MAX), as
//    the TensorRT-LLM page "Block-skip fast path for self-sampling GVR top-K
//    decode" (PR 18122) describes for its optional values output;
//  * optional sorting of each long row's K indices by value descending, then
//    index ascending ("optional output sorting", PR 20998 "What changes").
// One workgroup per row; the K (key, index) pairs are sorted in LDS with a
// bitonic network.  Reads only the row's window and the indices the
// selection wrote.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gvr_common.h"
#include "row_window.h"

namespace ert {

namespace {

// Order-preserving key with -0 folded into +0 (same map as the selection).
__device__ __forceinline__ uint32_t epi_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b >> 31) ? ~b : (b | 0x80000000u);
}

}  // namespace

template <int K>
__global__ void __launch_bounds__(kEpiBlock) topk_epilogue_kernel(const EpiParams p) {
  constexpr int BLOCK = kEpiBlock;
  __shared__ uint64_t s[K];
  const int t = threadIdx.x;
  const int64_t row = (int64_t)p.row_begin + blockIdx.x;
  const int S = (int)p.row_stride;
  int ks, nv;
  row_window(p.n_valid, p.row_starts, p.row_ends, p.varlen, row, S, &ks, &nv);
  int32_t* out = p.indices + row * K;
  float* vals = p.values ? p.values + row * K : nullptr;
  const float* win = p.logits + row * (int64_t)S + ks;
  const float lowest = -__FLT_MAX__;

  if (nv <= K) {
    // identity + -1: the values are the window itself, then the pad value
    if (vals)
      for (int i = t; i < K; i += BLOCK) vals[i] = i < nv ? win[i] : lowest;
    return;
  }
  if (!p.sorted) {
    if (vals)
      for (int i = t; i < K; i += BLOCK) {
        const int32_t idx = out[i];
        vals[i] = (idx >= 0 && idx < nv) ? win[idx] : lowest;
      }
    return;
  }
  // Sort descending on (key << 32) | ~index: value descending, then index
  // ascending.  Indices outside [0, nv) cannot come from the selection; they
  // sort last with the lowest key and are written back unchanged.
  for (int i = t; i < K; i += BLOCK) {
    const int32_t idx = out[i];
    const bool ok = idx >= 0 && idx < nv;
    const uint32_t key = ok ? epi_key(win[idx]) : 0u;
    s[i] = ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)idx);
  }
  __syncthreads();
  for (int size = 2; size <= K; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < K / 2; i += BLOCK) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const uint64_t a = s[lo], b = s[hi];
        // blocks of `size` alternate direction; the last merge is descending
        const bool desc = (lo & size) == 0;
        if (desc ? (a < b) : (a > b)) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = t; i < K; i += BLOCK) {
    const int32_t idx = (int32_t)(~(uint32_t)s[i]);
    out[i] = idx;
    if (vals) vals[i] = (idx >= 0 && idx < nv) ? win[idx] : lowest;
  }
}

const void* epilogue_kernel(int k) {
  switch (k) {
    case 512: return reinterpret_cast<const void*>(&topk_epilogue_kernel<512>);
    case 1024: return reinterpret_cast<const void*>(&topk_epilogue_kernel<1024>);
    case 2048: return reinterpret_cast<const void*>(&topk_epilogue_kernel<2048>);
    default: return nullptr;
  }
}

}  // namespace ert
