// gvr_common.h -- shapes and launch parameters shared by the gfx950 kernels and
// the C-ABI host code of the exact per-row top-K library.  Device-independent
// constants only; no HIP device code here.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ert {

// Value-histogram bins over the sampled bracket.  The pages do not state a bin
// count; 2048 keeps the crossing bin of a Gaussian-like row at tens of members
// for every K while the LDS histogram stays at 8 KiB.
constexpr int kBins = 2048;

// Candidate capacity held in LDS (one-workgroup tier, and the split tier's
// final refine).
constexpr int kSingleCap = 2048;

// Per-row candidate storage of the split tier (workspace).  The pages' rescue
// trigger is m > min(CS x 4096, 32 x K, 16384) with CS workgroups per row
// (PR 20998 "What changes"); 16384 is its ceiling.
constexpr int kSplitCapMax = 16384;
constexpr int kSplitCapPerWg = 4096;

// Split tier: a row whose sampled count above the floor bin predicts more
// than this many scores there goes straight to the parallel rescue.
constexpr int kPredictMax = kSplitCapMax / 2;

// Launch variants: (workgroup size, float4 groups per thread).
struct Variant {
  int block;
  int qpt;
};
// One workgroup per row; resident capacity block * qpt * 4 scores.
constexpr Variant kSingleVariants[] = {{256, 8}, {512, 9}, {1024, 9}};
// G workgroups per row, each holding 1/G of the row.
constexpr int kSplitBlock = 256;
constexpr int kSplitQpt[] = {4, 8, 17};

constexpr int kMaxWgsPerRow = 64;
constexpr int kMaxSlots = 256;  // split rows per launch (workspace slots)
constexpr int kStatsWords = 8;

// Workspace layout (bytes):
//   [0, 256)                             error flags (word 0)
//   kMaxSlots fixed blocks of 4352 bytes: SlotHeader + digit counts [4][256]
//   then one data block per slot: candidate (key, index) pairs
//   [kSplitCapMax]; consecutive blocks are skewed by 4 KiB so the slots'
//   first bytes do not all land on the same memory channels
// The fixed blocks hold every word that carries state between calls, and the
// last workgroup of a row returns them to zero (only the barrier generation
// keeps counting); their place does not depend on the plan, so one workspace
// serves any plan it is large enough for.  Data blocks are written before they
// are read and need no clearing.
struct SlotHeader {
  uint32_t bar_count;  // barrier arrivals (returns to 0 after each barrier)
  uint32_t bar_gen;    // barrier generation (monotone, never reset)
  uint32_t done;       // workgroups finished with the slot (last one cleans)
  uint32_t win_cur;    // winner output cursor
  uint32_t cand_cur;   // candidate cursor
  uint32_t tie_cur;    // tie tickets (rescue)
  uint32_t pad[58];    // header is 256 bytes
};
static_assert(sizeof(SlotHeader) == 256, "slot header size");

struct SlotFixed {
  SlotHeader hdr;
  uint32_t dig[4][256];  // rescue digit counts, one row per radix level
};
static_assert(sizeof(SlotFixed) == 4352, "slot fixed block size");

constexpr size_t kWsHeaderBytes = 256;
constexpr size_t kWsDataOff = kWsHeaderBytes + sizeof(SlotFixed) * kMaxSlots;
constexpr size_t kSlotDataBytes = 2 * sizeof(uint32_t) * kSplitCapMax + 4096;
constexpr size_t ws_bytes_for(int slots) { return kWsDataOff + (size_t)slots * kSlotDataBytes; }

// Error flags written by the kernel into workspace word 0.
constexpr uint32_t kErrBarrierTimeout = 1u;

struct GvrParams {
  const float* logits;
  int64_t row_stride;
  const int32_t* n_valid;     // decode form, or nullptr
  const int32_t* row_starts;  // prefill form
  const int32_t* row_ends;
  int32_t row_begin;  // first row handled by this launch
  int32_t rows;       // rows handled by this launch
  int32_t wgs_per_row;
  int32_t xcd_group;  // 1: map a row's workgroups onto one XCD
  int32_t cap;        // candidate cap of this plan
  int32_t force_rescue;
  int32_t* indices;
  int32_t* row_stats;  // optional
  unsigned char* ws;   // workspace base (split tier), or nullptr
};

}  // namespace ert
