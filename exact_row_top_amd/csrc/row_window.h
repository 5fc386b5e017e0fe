// row_window.h -- the row resolve step shared by the selection kernel and the
// output epilogue: a row's window [ks, ks + nv) inside its stride, with the
// boundary's clamps (decode: n_valid clamped to [0, stride]; prefill: ks and
// ke clamped to [0, stride], ke >= ks; varlen decode: the MTP window formula,
// then the same clamp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gvr_common.h"

namespace ert {

__device__ __forceinline__ void row_window(const int32_t* n_valid, const int32_t* row_starts,
                                           const int32_t* row_ends, const VarlenForm& vf,
                                           int64_t row, int S, int* ks, int* nv) {
  if (vf.kv_lens) {
    // row < 2^31 and next_n, compress_ratio >= 1 (checked on the host): the
    // quotients are 32-bit unsigned ones; with kv >= next_n the numerator
    // kv - next_n + row % next_n + 1 lies in [1, kv]
    const uint32_t r = (uint32_t)row, nn = (uint32_t)vf.next_n;
    const uint32_t req = r / nn;
    const int32_t kv = vf.kv_lens[req];
    int n = 0;
    if (kv >= vf.next_n) {
      const uint32_t t = (uint32_t)(kv - vf.next_n) + (r - req * nn) + 1u;
      n = (int)(t / (uint32_t)vf.compress_ratio);
    }
    *ks = 0;
    *nv = n > S ? S : n;
  } else if (n_valid) {
    const int n = n_valid[row];
    *ks = 0;
    *nv = n < 0 ? 0 : (n > S ? S : n);
  } else {
    int a = row_starts[row], e = row_ends[row];
    a = a < 0 ? 0 : (a > S ? S : a);
    e = e < a ? a : (e > S ? S : e);
    *ks = a;
    *nv = e - a;
  }
}

}  // namespace ert
