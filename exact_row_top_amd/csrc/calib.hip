// calib.hip -- a measurement aid, not part of the selection: the read floor
// of a batch.  One launch reads exactly the scores the selection reads (the
// windows of rows longer than K, as aligned float4 groups), with the launch
// shape the selection's plan uses (one workgroup per row, or G per row with
// the same part split and XCD renumbering), and folds them into one word per
// workgroup so the loads are not removed.  Its time is what the row reads
// alone cost in that shape: the floor under the selection's time.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gvr_common.h"
#include "gvr_device.h"
#include "row_window.h"

namespace ert {

template <int QPT, int BLOCK>
__global__ void __launch_bounds__(BLOCK) read_floor_kernel(const GvrParams p, int k, uint32_t* sink) {
  const int G = p.wgs_per_row;
  int slot, g;
  if (G > 1) {
    int L = blockIdx.x;
    if (p.xcd_group) {
      const int per = gridDim.x >> 3;
      L = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    }
    slot = L / G;
    g = L - slot * G;
  } else {
    slot = (int)gridDim.x - 1 - (int)blockIdx.x;
    g = 0;
  }
  if (slot >= p.rows) return;
  const int64_t row = (int64_t)p.row_begin + slot;
  const int S = (int)p.row_stride;
  int ks, nv;
  row_window(p.n_valid, p.row_starts, p.row_ends, p.varlen, row, S, &ks, &nv);
  if (nv <= k) return;
  const int Q = ((ks & 3) + nv + 3) >> 2;
  int q0 = 0, q1 = Q;
  if (G > 1) {
    const int Qp = (Q + G - 1) / G;
    q0 = g * Qp;
    q1 = q0 + Qp < Q ? q0 + Qp : Q;
  }
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int l = lane_id();
  const f4* base = reinterpret_cast<const f4*>(p.logits + row * (int64_t)S + (ks & ~3));
  const int qw0 = __builtin_amdgcn_readfirstlane(q0 + w * 64);
  const int nj = __builtin_amdgcn_readfirstlane(qw0 < q1 ? min((q1 - qw0 + BLOCK - 1) / BLOCK, QPT) : 0);
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, q1 * 16);
  const int vo = (qw0 + l) * 16;
  f4 v[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j)
    if (j < nj)
      v[j] = __builtin_bit_cast(
          f4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, vo + j * BLOCK * 16, 0, kCachePolicyNT));
  uint32_t acc = 0u;
#pragma unroll
  for (int j = 0; j < QPT; ++j)
    if (j < nj)
      acc ^= __float_as_uint(v[j][0]) ^ __float_as_uint(v[j][1]) ^ __float_as_uint(v[j][2]) ^
             __float_as_uint(v[j][3]);
  if (acc == 0x9E3779B9u) sink[0] = acc;  // (data-dependent: keeps the loads)
}

template <int QPT, int BLOCK>
static const void* rf() {
  return reinterpret_cast<const void*>(&read_floor_kernel<QPT, BLOCK>);
}

const void* read_floor_kernel_ptr(int block, int qpt) {
  if (block == 256 && qpt == 4) return rf<4, 256>();
  if (block == 256 && qpt == 8) return rf<8, 256>();
  if (block == 256 && qpt == 17) return rf<17, 256>();
  if (block == 512 && qpt == 9) return rf<9, 512>();
  if (block == 1024 && qpt == 9) return rf<9, 1024>();
  return nullptr;
}

}  // namespace ert
