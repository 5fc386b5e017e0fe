// topk_abi.cpp -- C ABI of the exact per-row top-K library: host-side
// validation (no device reads), launch planning, workspace ownership and the
// kernel launches.  The contract is documented in include/exact_row_top.h.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string.h>

#include "exact_row_top.h"
#include "gvr_common.h"

namespace ert {
const void* gvr_kernel(int k, int block, int qpt, bool split);
const void* epilogue_kernel(int k);
const void* blockskip_kernel(int k, bool self);
const void* block_max_kernel_ptr(bool vec);
hipError_t state_timeout_address(uint32_t** out);
hipError_t state_scratch_address(void** out);
const void* fill_zero_kernel_ptr();
const void* read_floor_kernel_ptr(int block, int qpt);
const void* status_read_kernel_ptr();
const void* status_reset_kernel_ptr();
}

using namespace ert;

namespace {

bool k_ok(int32_t k) { return k == 512 || k == 1024 || k == 2048; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Plan {
  int G = 1;        // workgroups per row
  int block = 256;  // workgroup size
  int qpt = 4;      // float4 groups per thread
  int rows_per_launch = 0;
  int launches = 0;
  size_t ws_bytes = 0;
  int cap = kSingleCap;  // candidate cap
  int xcd_group = 0;
};

// A window of env_len floats starting at any ks spans at most this many
// aligned float4 groups (lead <= 3 plus a partial last group).
int64_t quads_for(int64_t env_len) { return (env_len + 3 + 3) / 4; }

// Work to fill the chip: about 512 wave quartets (256-thread groups) in
// flight.
constexpr int64_t kFillUnits = 512;
// Split tier: the part size (float4 groups) the planner aims at.
constexpr int64_t kSplitPart = 2048;
// Compute units per XCD on MI355X (256 units in 8 XCDs).
constexpr int64_t kCusPerXcd = 32;

// Launch shape for (rows, envelope, k).  `capacity` = workgroups the device
// keeps resident at once for the split kernel (only the split tier needs its
// workgroups co-resident, for the rescue's row barriers).
int make_plan(int32_t num_rows, int64_t env_len, int32_t k, int32_t force_g, int64_t capacity,
              Plan* pl) {
  Plan p;
  const int64_t Qmax = quads_for(env_len < 1 ? 1 : env_len);
  // smallest one-workgroup variant that holds the window
  int single = -1;
  for (int i = 0; i < (int)(sizeof(kSingleVariants) / sizeof(kSingleVariants[0])); ++i)
    if ((int64_t)kSingleVariants[i].block * kSingleVariants[i].qpt >= Qmax) {
      single = i;
      break;
    }
  int G;
  if (force_g > 0) {
    if (force_g > kMaxWgsPerRow) return TOPK_EINVAL;
    G = force_g;
    if (G == 1 && single < 0) return TOPK_EINVAL;  // row does not fit one workgroup
  } else if (single >= 0 &&
             (int64_t)num_rows * (kSingleVariants[single].block / 256) >= kFillUnits) {
    G = 1;  // enough rows to fill the chip with whole rows
  } else if (single == 0) {
    G = 1;  // rows short enough for the smallest workgroup: splitting costs more
            // in cross-workgroup latency than it gains in bandwidth
  } else {
    // Parts of about kSplitPart float4 groups, but no more parts than fill
    // the chip (kFillUnits workgroups in all), and at least as many as the
    // largest part shape needs.
    // Measured on MI355X (cold launches): 8 rows x 262144 at K = 2048 run
    // 39.1 us with 32 parts of 2048 groups against 43.8 with 64 of 1024;
    // 8 rows x 114963 at K = 512 17.8-18.3 us with 8-16 parts against 20.5
    // with 33 small ones; 64 rows x 131072 keep 8 parts (more would need a
    // second launch or add merge work: 23.1 us at 12 parts, 21.9 at 8).
    const int64_t part_max =
        (int64_t)kSplitVariants[kNumSplit - 1].block * kSplitVariants[kNumSplit - 1].qpt;
    const int64_t g_min = (Qmax + part_max - 1) / part_max;
    const int64_t g_fill = (kFillUnits + num_rows - 1) / (num_rows > 0 ? num_rows : 1);
    const int64_t g_useful = (Qmax + kSplitPart - 1) / kSplitPart;
    int64_t gg = g_fill < g_useful ? g_fill : g_useful;
    // At most one part per compute unit of an XCD (kCusPerXcd units) for the
    // rows an XCD holds: a launch of eight or more rows maps each row's
    // workgroups onto one XCD, so a part then never shares a unit and the
    // row does not wait for a part that did (8 rows x 262144, K = 2048:
    // 36.5 us with 32 parts, 40.1 with 33); fewer rows spread their parts
    // over the XCDs, where the cap costs nothing (2 rows x 262144: 19.4 us
    // at 32 parts against 22.7 at 64).
    const int64_t g_xcd = kCusPerXcd / ((num_rows + 7) / 8);
    if (g_xcd >= g_min && gg > g_xcd) gg = g_xcd;
    if (gg > kMaxWgsPerRow) gg = kMaxWgsPerRow;  // larger parts then
    if (gg < g_min) gg = g_min;
    if (gg < 1) gg = 1;
    if (gg > kMaxWgsPerRow) return TOPK_EINVAL;  // row longer than the largest plan
    G = (int)gg;
  }
  p.G = G;
  if (G == 1) {
    if (single < 0) {
      // one part of the split kernel would need G > 1
      return TOPK_EINVAL;
    }
    p.block = kSingleVariants[single].block;
    p.qpt = kSingleVariants[single].qpt;
    p.rows_per_launch = num_rows;
    p.launches = num_rows > 0 ? 1 : 0;
    p.ws_bytes = 0;
    p.cap = one_wg_cap(k);
  } else {
    const int64_t per_part = (Qmax + G - 1) / G;
    int qpt = 0, block = 0;
    for (const Variant& sv : kSplitVariants)
      // parts over 1024 groups take the 512-thread shape (eight waves to
      // hide a part's latency, as measured above) rather than 256 x 8
      if ((int64_t)sv.block * sv.qpt >= per_part &&
          !(sv.block == 256 && sv.qpt == 8 && per_part > 1024)) {
        qpt = sv.qpt;
        block = sv.block;
        break;
      }
    if (qpt == 0) return TOPK_EINVAL;  // forced G too small for this row length
    p.block = block;
    p.qpt = qpt;
    int64_t rpl = capacity / G;
    if (rpl > kMaxSlots) rpl = kMaxSlots;
    if (rpl > num_rows) rpl = num_rows;
    if (rpl < 1) return TOPK_EINVAL;
    p.rows_per_launch = (int)rpl;
    p.launches = num_rows > 0 ? (int)((num_rows + rpl - 1) / rpl) : 0;
    // slots are padded to a multiple of 8 when a row's workgroups share an XCD
    p.xcd_group = (rpl >= 8) ? 1 : 0;
    int64_t slots = p.xcd_group ? ((rpl + 7) / 8) * 8 : rpl;
    if (p.xcd_group && (slots * G > capacity || slots > kMaxSlots)) {
      p.xcd_group = 0;
      slots = rpl;
    }
    p.ws_bytes = ws_bytes_for((int)slots, G);
    p.cap = kSingleCap;
  }
  *pl = p;
  return TOPK_OK;
}

// Workspace bytes independent of the device: the largest slot count any
// device could use (rows per launch is bounded by kMaxSlots and num_rows).
size_t ws_bytes_upper(int32_t num_rows, int64_t env_len, int32_t k, int32_t force_g) {
  Plan p;
  if (make_plan(num_rows, env_len, k, force_g, (int64_t)1 << 40, &p) != TOPK_OK) return 0;
  if (p.G == 1) return 0;
  int64_t rpl = num_rows < kMaxSlots ? num_rows : kMaxSlots;
  int64_t slots = ((rpl + 7) / 8) * 8;
  if (slots > kMaxSlots) slots = kMaxSlots;
  return ws_bytes_for((int)slots, p.G);
}

int validate(int mode, const void* logits, int64_t row_stride, const void* e1, const void* e2,
             int32_t num_rows, int32_t k, const void* indices, int32_t force_g) {
  if (num_rows < 0 || !k_ok(k) || row_stride < 1 || row_stride >= ((int64_t)1 << 30) ||
      force_g < 0 || force_g > kMaxWgsPerRow)
    return TOPK_EINVAL;
  if (num_rows == 0) return TOPK_OK;
  if (!logits || !indices || !e1 || (mode == 1 && !e2)) return TOPK_EINVAL;
  if (!aligned(logits, 16) || (row_stride % 4) != 0) return TOPK_ELAYOUT;
  if (!aligned(indices, 4) || !aligned(e1, 4) || (mode == 1 && !aligned(e2, 4))) return TOPK_ELAYOUT;
  return TOPK_OK;
}

// ---- per-device facts ------------------------------------------------------
struct DevInfo {
  bool probed = false;
  bool ok = false;
  int cus = 0;
  int occ[3][kNumSplit] = {};      // [k idx][split variant] split-kernel workgroups per CU
  int occ_api[3][kNumSplit] = {};  // what hipOccupancyMaxActiveBlocksPerMultiprocessor says
  int regs[3][kNumSplit] = {};     // VGPRs per thread of each split kernel
  int lds[3][kNumSplit] = {};      // static LDS bytes
  void* slab = nullptr;
  size_t slab_bytes = 0;
  uint32_t* timeout = nullptr;  // this GPU's row-barrier timeout count
  void* scratch = nullptr;      // this GPU's fixed workspace (topk_decode_noalloc)
  bool scratch_cleared = false;
};
constexpr int kMaxDev = 64;
DevInfo g_dev[kMaxDev];
std::mutex g_mu;

int kidx(int k) { return k == 512 ? 0 : (k == 1024 ? 1 : 2); }
int qidx(int q) {
  for (int i = 0; i < kNumSplit; ++i)
    if (kSplitVariants[i].qpt == q) return i;
  return 0;
}

int device_info(DevInfo** out, int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return TOPK_EDEVICE;
  DevInfo& d = g_dev[dev];
  if (!d.probed) {
    d.probed = true;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TOPK_EDEVICE;
    d.ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    // set-up, with this device current: its copies of the library's device
    // variables (the host-side names are stand-ins, never device addresses)
    if (d.ok && (state_timeout_address(&d.timeout) != hipSuccess || !d.timeout ||
                 state_scratch_address(&d.scratch) != hipSuccess || !d.scratch))
      d.ok = false;
    for (int ki = 0; ki < 3; ++ki)
      for (int qi = 0; qi < kNumSplit; ++qi) {
        const int ks[3] = {512, 1024, 2048};
        const int blk = kSplitVariants[qi].block;
        const void* f = gvr_kernel(ks[ki], blk, kSplitVariants[qi].qpt, true);
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, blk, 0) != hipSuccess)
          nb = 0;
        d.occ_api[ki][qi] = nb;
        // Residency from the kernel's own resources and the gfx950 compute
        // unit: 4 SIMDs with 512 VGPRs per lane each (granule 8), at most 8
        // waves per SIMD, 160 KiB of LDS.  Taken as the smaller of this and
        // the runtime's figure when the latter is available, so the split
        // tier never plans more co-resident workgroups than both allow.
        hipFuncAttributes at;
        int mine = 1;
        if (hipFuncGetAttributes(&at, f) == hipSuccess) {
          const int v = at.numRegs > 0 ? ((at.numRegs + 7) / 8) * 8 : 512;
          const int waves_simd = std::min(8, 512 / v);
          const int wg_waves = blk / 64;
          const int by_vgpr = (4 * waves_simd) / wg_waves;
          const int lds = (int)at.sharedSizeBytes;
          const int by_lds = lds > 0 ? (160 * 1024) / lds : 64;
          mine = std::max(1, std::min(by_vgpr, by_lds));
          d.regs[ki][qi] = at.numRegs;
          d.lds[ki][qi] = lds;
        }
        d.occ[ki][qi] = (nb > 0) ? std::min(nb, mine) : mine;
      }
  }
  if (!d.ok) return TOPK_EDEVICE;
  *out = &d;
  *dev_out = dev;
  return TOPK_OK;
}

// Shape-only gate of the block-skip pass (PR 18122 "Description"): the batch's
// padded working set reaches 128 MiB and rows are long against K (the row
// stride stands for the row length: no data-dependent term).
bool blockskip_gate(int32_t num_rows, int64_t row_stride, int32_t k) {
  return (int64_t)num_rows * row_stride * 4 >= ((int64_t)128 << 20) && row_stride >= (int64_t)72 * k;
}

// Streaming tier (the block-skip pass making its own maxima) for batches of
// many long decode rows: at least 128 rows, rows longer than one resident
// workgroup holds and at least 4 K whole blocks of 32 per row (so the K-th
// largest block maximum gives the floor), up to the pass's 8192 blocks.
// Measured on MI355X against the resident tiers (i.i.d. rows; rows with
// locality gain 2-4x more): 128 x 131072 K=512 32.8 vs 35.5 us, 1024 x 65536
// K=512 101 vs 123 us, 512 x 131072 K=512 71 vs 136 us, 256 x 262144 K=2048
// 86 vs 135 us; shapes it loses on (256 x 65536 K=1024, 512 x 65536 K=2048,
// 256 x 131072 K=2048) fail the 4 K blocks rule.
bool stream_gate(int32_t num_rows, int64_t row_stride, int32_t k) {
  const int64_t single_max = (int64_t)kSingleVariants[3].block * kSingleVariants[3].qpt * 4;
  return num_rows >= 128 && row_stride > single_max && row_stride / 32 >= (int64_t)4 * k &&
         (row_stride + 31) / 32 <= kBskMaxBlocks;
}

// Output stage after the selection: values and / or sorted long rows.
int launch_epilogue(const GvrParams& prm, int32_t k, int32_t num_rows, float* values,
                    uint32_t flags, hipStream_t stream) {
  if (values || (flags & TOPK_SORTED)) {
    // output stage: values and / or sorted long rows, one workgroup per row
    const void* epi = epilogue_kernel(k);
    if (!epi) return TOPK_EINVAL;
    EpiParams ep;
    memset(&ep, 0, sizeof(ep));
    ep.logits = prm.logits;
    ep.row_stride = prm.row_stride;
    ep.n_valid = prm.n_valid;
    ep.row_starts = prm.row_starts;
    ep.row_ends = prm.row_ends;
    ep.varlen = prm.varlen;
    ep.sorted = (flags & TOPK_SORTED) ? 1 : 0;
    ep.indices = prm.indices;
    ep.values = values;
    constexpr int64_t kMaxGrid = (int64_t)1 << 30;
    for (int64_t r0 = 0; r0 < num_rows; r0 += kMaxGrid) {
      const int64_t nr = (num_rows - r0) < kMaxGrid ? (num_rows - r0) : kMaxGrid;
      ep.row_begin = (int32_t)r0;
      void* args[] = {&ep};
      if (hipLaunchKernel(epi, dim3((unsigned)nr), dim3(kEpiBlock), args, 0, stream) != hipSuccess)
        return TOPK_ELAUNCH;
    }
  }
  if (hipGetLastError() != hipSuccess) return TOPK_ELAUNCH;
  return TOPK_OK;
}

int run(int mode, const float* logits, int64_t row_stride, const int32_t* e1, const int32_t* e2,
        int32_t num_rows, int32_t k, int32_t* indices, int64_t max_row_len, void* workspace,
        size_t workspace_bytes, hipStream_t stream, const topk_options* opts,
        const VarlenForm* vf = nullptr, bool use_scratch = false) {
  const int32_t force_g = opts ? opts->force_wgs_per_row : 0;
  int rc = validate(mode, logits, row_stride, e1, e2, num_rows, k, indices, force_g);
  if (rc != TOPK_OK) return rc;
  if (vf && num_rows > 0 && (vf->next_n < 1 || vf->compress_ratio < 1)) return TOPK_EINVAL;
  if (opts && opts->row_stats && !aligned(opts->row_stats, 4)) return TOPK_ELAYOUT;
  const uint32_t flags = opts ? opts->flags : 0u;
  float* values = opts ? opts->values : nullptr;
  if (flags & ~(uint32_t)(TOPK_SORTED | TOPK_DETERMINISTIC)) return TOPK_EINVAL;
  if (values && !aligned(values, 4)) return TOPK_ELAYOUT;
  const int32_t* hints = opts ? opts->pre_idx : nullptr;
  if (hints) {
    if (mode != 0) return TOPK_EINVAL;  // the prefill form takes no hints
    if (opts->pre_idx_stride < k) return TOPK_EINVAL;
    if (!aligned(hints, 4)) return TOPK_ELAYOUT;
  }
  const float* bmax = opts ? opts->bmax : nullptr;
  const int32_t bsk_mode = opts ? opts->blockskip : 0;
  if (bsk_mode < -1 || bsk_mode > 2) return TOPK_EINVAL;
  if (opts && opts->barrier_spins < 0) return TOPK_EINVAL;
  if (bsk_mode == 2 && (mode != 0 || (row_stride + 31) / 32 > kBskMaxBlocks)) return TOPK_EINVAL;
  if (bmax) {
    if (mode != 0) return TOPK_EINVAL;  // block-skip serves the decode forms
    if (opts->bmax_stride < (row_stride + 31) / 32) return TOPK_EINVAL;
    if (!aligned(bmax, 4)) return TOPK_ELAYOUT;
  } else if (bsk_mode == 1) {
    return TOPK_EINVAL;  // forced block-skip needs block maxima
  }
  if (num_rows == 0) return TOPK_OK;
  // Plans are sized for the full row stride, so any window inside it fits the
  // resident capacity; the prefill length hint is accepted but not needed.
  if (max_row_len < 0) return TOPK_EINVAL;
  const int64_t env = row_stride;

  std::lock_guard<std::mutex> lock(g_mu);
  DevInfo* d = nullptr;
  int dev = 0;
  rc = device_info(&d, &dev);
  if (rc != TOPK_OK) return rc;

  if (use_scratch) {
    // the fixed per-device scratch stands in for the workspace: nothing is
    // allocated; its first use on this device clears it with a kernel on the
    // caller's stream (the array rests at zero between calls after that)
    workspace = d->scratch;
    workspace_bytes = kScratchBytes;
    if (!d->scratch_cleared) {
      uint4* p = static_cast<uint4*>(d->scratch);
      size_t n = kScratchBytes / 16;
      void* a[] = {&p, &n};
      if (hipLaunchKernel(fill_zero_kernel_ptr(), dim3(256), dim3(256), a, 0, stream) != hipSuccess)
        return TOPK_ELAUNCH;
      d->scratch_cleared = true;
    }
  }

  GvrParams prm;
  memset(&prm, 0, sizeof(prm));
  prm.logits = logits;
  prm.row_stride = row_stride;
  prm.n_valid = (mode == 0 && !vf) ? e1 : nullptr;
  prm.row_starts = (mode == 1) ? e1 : nullptr;
  prm.row_ends = (mode == 1) ? e2 : nullptr;
  if (vf) prm.varlen = VarlenForm{e1, vf->next_n, vf->compress_ratio};
  prm.force_rescue = (opts && opts->force_rescue) ? 1 : 0;
  prm.deterministic = (flags & TOPK_DETERMINISTIC) ? 1 : 0;
  prm.indices = indices;
  prm.row_stats = opts ? opts->row_stats : nullptr;
  prm.sync.err = d->timeout;
  prm.sync.spins = (opts && opts->barrier_spins > 0) ? (uint32_t)opts->barrier_spins : kDefaultSpins;

  const bool given = bmax && bsk_mode >= 0 &&
                     (bsk_mode == 1 || blockskip_gate(num_rows, row_stride, k));
  const bool self = !given && (bsk_mode == 2 || (mode == 0 && bsk_mode == 0 && force_g == 0 &&
                                                 !(opts && opts->force_rescue) &&
                                                 stream_gate(num_rows, row_stride, k)));
  if (given || self) {
    // block-skip pass: one 1024-thread workgroup per row, no workspace; the
    // streaming form reads every block once and makes the maxima itself
    const void* kern = blockskip_kernel(k, self);
    if (!kern) return TOPK_EINVAL;
    prm.wgs_per_row = 1;
    prm.rows = num_rows;
    prm.row_begin = 0;
    int64_t bstride = given ? opts->bmax_stride : 0;  // opts may be null here
    void* args[] = {&prm, &bmax, &bstride};
    if (hipLaunchKernel(kern, dim3((unsigned)num_rows), dim3(1024), args, 0, stream) != hipSuccess)
      return TOPK_ELAUNCH;
    return launch_epilogue(prm, k, num_rows, values, flags, stream);
  }

  // The plan's first guess may be for a single workgroup per row; the split
  // capacity is only consulted when G > 1.
  Plan pl;
  rc = make_plan(num_rows, env, k, force_g, (int64_t)1 << 40, &pl);
  if (rc != TOPK_OK) return rc;
  if (pl.G > 1) {
    const int64_t cap = (int64_t)d->cus * d->occ[kidx(k)][qidx(pl.qpt)];
    rc = make_plan(num_rows, env, k, force_g, cap, &pl);
    if (rc != TOPK_OK) return rc;
  }

  unsigned char* ws = nullptr;
  if (pl.G > 1) {
    if (workspace) {
      if (!aligned(workspace, 16)) return TOPK_ELAYOUT;
      if (workspace_bytes < pl.ws_bytes) return TOPK_EWORKSPACE;
      ws = static_cast<unsigned char*>(workspace);
    } else {
      const size_t need = ws_bytes_upper(num_rows, env, k, force_g);
      const size_t want = need > pl.ws_bytes ? need : pl.ws_bytes;
      if (d->slab_bytes < want) {
        if (d->slab) {
          if (hipDeviceSynchronize() != hipSuccess) return TOPK_ELAUNCH;
          (void)hipFree(d->slab);
          d->slab = nullptr;
          d->slab_bytes = 0;
        }
        // zeroed before any stream can use it: the memset completes before
        // the call returns (allocation is not capture-safe either way)
        void* ptr = nullptr;
        if (hipMalloc(&ptr, want) != hipSuccess) return TOPK_ELAUNCH;
        if (hipMemsetAsync(ptr, 0, want, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess) {
          (void)hipFree(ptr);
          return TOPK_ELAUNCH;
        }
        d->slab = ptr;
        d->slab_bytes = want;
      }
      ws = static_cast<unsigned char*>(d->slab);
    }
  }

  const void* kern = gvr_kernel(k, pl.block, pl.qpt, pl.G > 1);
  if (!kern) return TOPK_EINVAL;
  prm.wgs_per_row = pl.G;
  prm.cap = pl.cap;
  prm.hints = hints;
  prm.hint_stride = hints ? opts->pre_idx_stride : 0;
  prm.hint_div = vf ? vf->next_n : 1;  // hints are per request
  prm.ws = ws;
  for (int64_t r0 = 0; r0 < num_rows; r0 += pl.rows_per_launch) {
    const int64_t nr = (num_rows - r0) < pl.rows_per_launch ? (num_rows - r0) : pl.rows_per_launch;
    prm.row_begin = (int32_t)r0;
    prm.rows = (int32_t)nr;
    int64_t grid;
    if (pl.G == 1) {
      prm.xcd_group = 0;
      grid = nr;
    } else {
      prm.xcd_group = (pl.xcd_group && nr >= 8) ? 1 : 0;
      grid = prm.xcd_group ? ((nr + 7) / 8) * 8 * pl.G : nr * pl.G;
    }
    void* args[] = {&prm};
    if (hipLaunchKernel(kern, dim3((unsigned)grid), dim3(pl.block), args, 0, stream) != hipSuccess)
      return TOPK_ELAUNCH;
  }
  return launch_epilogue(prm, k, num_rows, values, flags, stream);
}

}  // namespace

extern "C" {

int topk_decode(const float* logits, int64_t row_stride, const int32_t* n_valid, int32_t num_rows,
                int32_t k, int32_t* indices, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  return run(0, logits, row_stride, n_valid, nullptr, num_rows, k, indices, 0, workspace,
             workspace_bytes, stream, nullptr);
}

int topk_prefill(const float* logits, int64_t row_stride, const int32_t* row_starts,
                 const int32_t* row_ends, int32_t num_rows, int32_t k, int32_t* indices,
                 int64_t max_row_len, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(1, logits, row_stride, row_starts, row_ends, num_rows, k, indices, max_row_len,
             workspace, workspace_bytes, stream, nullptr);
}

int topk_decode_noalloc(const float* logits, int64_t row_stride, const int32_t* n_valid,
                        int32_t num_rows, int32_t k, int32_t* indices, hipStream_t stream) {
  return run(0, logits, row_stride, n_valid, nullptr, num_rows, k, indices, 0, nullptr, 0, stream,
             nullptr, nullptr, true);
}

int topk_decode_v(const float* logits, int64_t row_stride, const int32_t* n_valid,
                  int32_t num_rows, int32_t k, int32_t* indices, float* values, uint32_t flags,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  topk_options o;
  memset(&o, 0, sizeof(o));
  o.values = values;
  o.flags = flags;
  return run(0, logits, row_stride, n_valid, nullptr, num_rows, k, indices, 0, workspace,
             workspace_bytes, stream, &o);
}

int topk_prefill_v(const float* logits, int64_t row_stride, const int32_t* row_starts,
                   const int32_t* row_ends, int32_t num_rows, int32_t k, int32_t* indices,
                   float* values, uint32_t flags, int64_t max_row_len, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  topk_options o;
  memset(&o, 0, sizeof(o));
  o.values = values;
  o.flags = flags;
  return run(1, logits, row_stride, row_starts, row_ends, num_rows, k, indices, max_row_len,
             workspace, workspace_bytes, stream, &o);
}

int topk_decode_varlen(const float* logits, int64_t row_stride, const int32_t* kv_lens,
                       int32_t num_rows, int32_t next_n, int32_t compress_ratio, int32_t k,
                       int32_t* indices, float* values, uint32_t flags, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  topk_options o;
  memset(&o, 0, sizeof(o));
  o.values = values;
  o.flags = flags;
  const VarlenForm vf{kv_lens, next_n, compress_ratio};
  return run(0, logits, row_stride, kv_lens, nullptr, num_rows, k, indices, 0, workspace,
             workspace_bytes, stream, &o, &vf);
}

int topk_decode_hinted(const float* logits, int64_t row_stride, const int32_t* n_valid,
                       const int32_t* pre_idx, int64_t pre_idx_stride, int32_t num_rows, int32_t k,
                       int32_t* indices, float* values, uint32_t flags, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  topk_options o;
  memset(&o, 0, sizeof(o));
  o.values = values;
  o.flags = flags;
  o.pre_idx = pre_idx;
  o.pre_idx_stride = pre_idx_stride;
  return run(0, logits, row_stride, n_valid, nullptr, num_rows, k, indices, 0, workspace,
             workspace_bytes, stream, &o);
}

int topk_decode_varlen_hinted(const float* logits, int64_t row_stride, const int32_t* kv_lens,
                              const int32_t* pre_idx, int64_t pre_idx_stride, int32_t num_rows,
                              int32_t next_n, int32_t compress_ratio, int32_t k, int32_t* indices,
                              float* values, uint32_t flags, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  topk_options o;
  memset(&o, 0, sizeof(o));
  o.values = values;
  o.flags = flags;
  o.pre_idx = pre_idx;
  o.pre_idx_stride = pre_idx_stride;
  const VarlenForm vf{kv_lens, next_n, compress_ratio};
  return run(0, logits, row_stride, kv_lens, nullptr, num_rows, k, indices, 0, workspace,
             workspace_bytes, stream, &o, &vf);
}

int topk_block_max(const float* logits, int64_t row_stride, int32_t num_rows, float* bmax,
                   int64_t bmax_stride, hipStream_t stream) {
  if (num_rows < 0 || row_stride < 1 || row_stride >= ((int64_t)1 << 30)) return TOPK_EINVAL;
  if (num_rows == 0) return TOPK_OK;
  if (!logits || !bmax) return TOPK_EINVAL;
  const int64_t nb = (row_stride + 31) / 32;
  if (bmax_stride < nb) return TOPK_EINVAL;
  if (!aligned(logits, 4) || !aligned(bmax, 4)) return TOPK_ELAYOUT;
  // coalesced 16-byte loads (eight lanes per block) when the layout allows
  const bool vec = aligned(logits, 16) && (row_stride % 4) == 0;
  const int64_t total = (int64_t)num_rows * nb;
  const int64_t per_wg = vec ? 32 : 256;  // blocks of 32 per workgroup of 256
  const int64_t grid = (total + per_wg - 1) / per_wg;
  if (grid >= ((int64_t)1 << 31)) return TOPK_EINVAL;
  int32_t nr = num_rows;
  void* args[] = {const_cast<float**>(&logits), &row_stride, &nr, &bmax, &bmax_stride};
  if (hipLaunchKernel(block_max_kernel_ptr(vec), dim3((unsigned)grid), dim3(256), args, 0,
                      stream) != hipSuccess)
    return TOPK_ELAUNCH;
  if (hipGetLastError() != hipSuccess) return TOPK_ELAUNCH;
  return TOPK_OK;
}

int topk_decode_blockskip(const float* logits, int64_t row_stride, const int32_t* n_valid,
                          const float* bmax, int64_t bmax_stride, int32_t num_rows, int32_t k,
                          int32_t* indices, float* values, uint32_t flags, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  topk_options o;
  memset(&o, 0, sizeof(o));
  o.values = values;
  o.flags = flags;
  o.bmax = bmax;
  o.bmax_stride = bmax_stride;
  if (!bmax && num_rows > 0) return TOPK_EINVAL;
  return run(0, logits, row_stride, n_valid, nullptr, num_rows, k, indices, 0, workspace,
             workspace_bytes, stream, &o);
}

int topk_decode_varlen_ex(const float* logits, int64_t row_stride, const int32_t* kv_lens,
                          int32_t num_rows, int32_t next_n, int32_t compress_ratio, int32_t k,
                          int32_t* indices, void* workspace, size_t workspace_bytes,
                          hipStream_t stream, const topk_options* opts) {
  const VarlenForm vf{kv_lens, next_n, compress_ratio};
  return run(0, logits, row_stride, kv_lens, nullptr, num_rows, k, indices, 0, workspace,
             workspace_bytes, stream, opts, &vf);
}

int topk_decode_ex(const float* logits, int64_t row_stride, const int32_t* n_valid,
                   int32_t num_rows, int32_t k, int32_t* indices, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, const topk_options* opts) {
  return run(0, logits, row_stride, n_valid, nullptr, num_rows, k, indices, 0, workspace,
             workspace_bytes, stream, opts);
}

int topk_prefill_ex(const float* logits, int64_t row_stride, const int32_t* row_starts,
                    const int32_t* row_ends, int32_t num_rows, int32_t k, int32_t* indices,
                    int64_t max_row_len, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, const topk_options* opts) {
  return run(1, logits, row_stride, row_starts, row_ends, num_rows, k, indices, max_row_len,
             workspace, workspace_bytes, stream, opts);
}

size_t topk_workspace_bytes(int32_t num_rows, int64_t max_row_len, int32_t k) {
  if (num_rows < 0 || !k_ok(k) || max_row_len < 1) return 0;
  if (num_rows == 0) return 0;
  return ws_bytes_upper(num_rows, max_row_len, k, 0);
}

int topk_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace && workspace_bytes) return TOPK_EINVAL;
  if (!workspace_bytes) return TOPK_OK;
  return hipMemsetAsync(workspace, 0, workspace_bytes, stream) == hipSuccess ? TOPK_OK
                                                                              : TOPK_ELAUNCH;
}

int topk_status(int32_t* timeouts, hipStream_t stream) {
  if (!timeouts) return TOPK_EINVAL;
  if (!aligned(timeouts, 4)) return TOPK_ELAYOUT;
  std::lock_guard<std::mutex> lock(g_mu);
  DevInfo* d = nullptr;
  int dev = 0;
  const int rc = device_info(&d, &dev);
  if (rc != TOPK_OK) return rc;
  uint4* slab = static_cast<uint4*>(d->slab);
  size_t n0 = d->slab_bytes / 16;
  uint4* scr = static_cast<uint4*>(d->scratch);
  size_t n1 = d->scratch_cleared ? kScratchBytes / 16 : 0;
  void* a1[] = {&d->timeout, &timeouts, &slab, &n0, &scr, &n1};
  if (hipLaunchKernel(status_read_kernel_ptr(), dim3(256), dim3(256), a1, 0, stream) != hipSuccess)
    return TOPK_ELAUNCH;
  void* a2[] = {&d->timeout};
  if (hipLaunchKernel(status_reset_kernel_ptr(), dim3(1), dim3(64), a2, 0, stream) != hipSuccess)
    return TOPK_ELAUNCH;
  return hipGetLastError() == hipSuccess ? TOPK_OK : TOPK_ELAUNCH;
}

const char* topk_strerror(int status) {
  switch (status) {
    case TOPK_OK: return "ok";
    case TOPK_EINVAL: return "invalid argument (null pointer, num_rows < 0, k not in {512,1024,2048}, row_stride < 1, or row too long)";
    case TOPK_ELAYOUT: return "unsupported layout (logits and workspace must be 16-byte aligned with row_stride % 4 == 0; indices/extents 4-byte aligned)";
    case TOPK_EWORKSPACE: return "workspace smaller than topk_workspace_bytes()";
    case TOPK_EDEVICE: return "current device is not gfx950";
    case TOPK_ELAUNCH: return "HIP launch or allocation failed";
    default: return "unknown status";
  }
}

int topk_read_floor(int32_t mode, const float* logits, int64_t row_stride, const int32_t* extents,
                    const int32_t* extents2, int32_t num_rows, int32_t k, uint32_t* sink,
                    hipStream_t stream) {
  if (mode != 0 && mode != 1) return TOPK_EINVAL;
  int rc = validate(mode, logits, row_stride, extents, extents2, num_rows, k, sink, 0);
  if (rc != TOPK_OK || num_rows == 0) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  DevInfo* d = nullptr;
  int dev = 0;
  rc = device_info(&d, &dev);
  if (rc != TOPK_OK) return rc;
  // the plan the selection would take (block-skip and streaming forms aside)
  Plan pl;
  rc = make_plan(num_rows, row_stride, k, 0, (int64_t)1 << 40, &pl);
  if (rc != TOPK_OK) return rc;
  if (pl.G > 1) {
    const int64_t cap = (int64_t)d->cus * d->occ[kidx(k)][qidx(pl.qpt)];
    rc = make_plan(num_rows, row_stride, k, 0, cap, &pl);
    if (rc != TOPK_OK) return rc;
  }
  const void* kern = read_floor_kernel_ptr(pl.block, pl.qpt);
  if (!kern) return TOPK_EINVAL;
  GvrParams prm;
  memset(&prm, 0, sizeof(prm));
  prm.logits = logits;
  prm.row_stride = row_stride;
  prm.n_valid = mode == 0 ? extents : nullptr;
  prm.row_starts = mode == 1 ? extents : nullptr;
  prm.row_ends = mode == 1 ? extents2 : nullptr;
  prm.wgs_per_row = pl.G;
  int32_t kk = k;
  for (int64_t r0 = 0; r0 < num_rows; r0 += pl.rows_per_launch) {
    const int64_t nr = (num_rows - r0) < pl.rows_per_launch ? (num_rows - r0) : pl.rows_per_launch;
    prm.row_begin = (int32_t)r0;
    prm.rows = (int32_t)nr;
    int64_t grid;
    if (pl.G == 1) {
      prm.xcd_group = 0;
      grid = nr;
    } else {
      prm.xcd_group = (pl.xcd_group && nr >= 8) ? 1 : 0;
      grid = prm.xcd_group ? ((nr + 7) / 8) * 8 * pl.G : nr * pl.G;
    }
    void* args[] = {&prm, &kk, &sink};
    if (hipLaunchKernel(kern, dim3((unsigned)grid), dim3(pl.block), args, 0, stream) != hipSuccess)
      return TOPK_ELAUNCH;
  }
  return hipGetLastError() == hipSuccess ? TOPK_OK : TOPK_ELAUNCH;
}

int topk_plan_query(int32_t num_rows, int64_t row_stride, int64_t max_row_len, int32_t k,
                    int32_t force_wgs_per_row, int32_t cu_count, int32_t wgs_per_cu, int64_t* out) {
  if (!out || num_rows < 0 || !k_ok(k) || row_stride < 1 || cu_count < 1 || wgs_per_cu < 1)
    return TOPK_EINVAL;
  if (max_row_len < 0) return TOPK_EINVAL;
  const int64_t env = row_stride;
  Plan pl;
  int rc = make_plan(num_rows, env, k, force_wgs_per_row, (int64_t)cu_count * wgs_per_cu, &pl);
  if (rc != TOPK_OK) return rc;
  out[0] = pl.G;
  out[1] = pl.qpt;
  out[2] = pl.rows_per_launch;
  out[3] = pl.launches;
  out[4] = (int64_t)pl.ws_bytes;
  out[5] = pl.cap;
  out[6] = pl.block;
  return TOPK_OK;
}

int topk_device_query(int64_t* out) {
  if (!out) return TOPK_EINVAL;
  std::lock_guard<std::mutex> lock(g_mu);
  DevInfo* d = nullptr;
  int dev = 0;
  const int rc = device_info(&d, &dev);
  if (rc != TOPK_OK) return rc;
  static_assert(kNumSplit == 3, "the query's layout holds three split variants");
  out[0] = d->cus;
  for (int ki = 0; ki < 3; ++ki)
    for (int qi = 0; qi < kNumSplit; ++qi) {
      out[1 + ki * 3 + qi] = d->occ[ki][qi];
      out[10 + ki * 3 + qi] = d->occ_api[ki][qi];
      out[19 + ki * 3 + qi] = d->regs[ki][qi];
      out[28 + ki * 3 + qi] = d->lds[ki][qi];
    }
  return TOPK_OK;
}

int topk_workspace_layout(int64_t* out) {
  if (!out) return TOPK_EINVAL;
  out[0] = (int64_t)kWsHeaderBytes;
  out[1] = (int64_t)sizeof(SlotFixed);
  out[2] = kMaxSlots;
  out[3] = (int64_t)kWsDataOff;
  out[4] = (int64_t)kSliceBytes;
  out[5] = (int64_t)kListBytes;
  return TOPK_OK;
}

int topk_validate(int32_t mode, const void* logits, int64_t row_stride, const void* extents,
                  const void* extents2, int32_t num_rows, int32_t k, const void* indices,
                  const void* workspace, size_t workspace_bytes, int64_t max_row_len) {
  if (mode != 0 && mode != 1) return TOPK_EINVAL;
  int rc = validate(mode, logits, row_stride, extents, extents2, num_rows, k, indices, 0);
  if (rc != TOPK_OK || num_rows == 0) return rc;
  if (max_row_len < 0) return TOPK_EINVAL;
  const int64_t env = row_stride;
  if (workspace) {
    Plan pl;
    rc = make_plan(num_rows, env, k, 0, (int64_t)1 << 40, &pl);
    if (rc != TOPK_OK) return rc;
    if (pl.G > 1 && !aligned(workspace, 16)) return TOPK_ELAYOUT;
    if (pl.G > 1 && workspace_bytes < ws_bytes_upper(num_rows, env, k, 0)) return TOPK_EWORKSPACE;
  }
  return TOPK_OK;
}

}  // extern "C"
