// gvr_common.h -- shapes and launch parameters shared by the gfx950 kernels and
// the C-ABI host code of the exact per-row top-K library.  Device-independent
// constants only; no HIP device code here.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ert {

// Workgroup: four wave64s.
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

// Value-histogram bins over the sampled bracket.  The pages do not state a bin
// count; 2048 keeps the crossing bin of a Gaussian-like row at tens of members
// for every K while the LDS histogram stays at 8 KiB.
constexpr int kBins = 2048;

// Candidate capacity of the one-workgroup tier (LDS, shares storage with the
// histogram once the crossing bin is known).
constexpr int kSingleCap = 2048;

// Per-row candidate storage of the split tier (workspace).  The pages' rescue
// trigger is m > min(CS x 4096, 32 x K, 16384) with CS workgroups per row
// (PR 20998 "What changes"); 16384 is its ceiling.
constexpr int kSplitCapMax = 16384;
constexpr int kSplitCapPerWg = 4096;

// Quads (float4 groups) per thread the kernels are instantiated for.
constexpr int kQptList[] = {4, 8, 17};
constexpr int kQptMax = 17;

constexpr int kMaxWgsPerRow = 64;
constexpr int kMaxSlots = 256;  // split rows per launch (workspace slots)
constexpr int kStatsWords = 8;

// Workspace layout: a 256-byte header, then kMaxSlots-bounded slots.
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

constexpr size_t kWsHeaderBytes = 256;  // word 0: error flags
constexpr size_t kSlotHistOff = sizeof(SlotHeader);
constexpr size_t kSlotDigitOff = kSlotHistOff + sizeof(uint32_t) * kBins;
constexpr size_t kSlotKeyOff = kSlotDigitOff + sizeof(uint32_t) * 4 * 256;
constexpr size_t kSlotIdxOff = kSlotKeyOff + sizeof(uint32_t) * kSplitCapMax;
constexpr size_t kSlotBytes = kSlotIdxOff + sizeof(int32_t) * kSplitCapMax;

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
