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

// Workspace layout (bytes):
//   [0, 256)                          error flags (word 0)
//   [256, 256 + kMaxSlots * 256)      one SlotHeader per split row of a launch
//   then, per slot, a data block of slot_data_bytes(G):
//     candidate keys [kSplitCapMax] | candidate indices [kSplitCapMax] |
//     per-workgroup histograms [G][kBins] | per-workgroup digit counts [G][4][256]
// Only the headers hold state between calls, and the last workgroup of a row
// returns its header to zero; their place does not depend on the plan, so
// one workspace serves any plan it is large enough for.  Data blocks are
// written densely before they are read and need no clearing.
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

constexpr size_t kWsHeaderBytes = 256;
constexpr size_t kWsSlotHeadersBytes = sizeof(SlotHeader) * kMaxSlots;
constexpr size_t kWsDataOff = kWsHeaderBytes + kWsSlotHeadersBytes;
constexpr size_t kSlotKeyOff = 0;
constexpr size_t kSlotIdxOff = kSlotKeyOff + sizeof(uint32_t) * kSplitCapMax;
constexpr size_t kSlotWgHistOff = kSlotIdxOff + sizeof(int32_t) * kSplitCapMax;
constexpr size_t slot_data_bytes(int wgs_per_row) {
  return kSlotWgHistOff + sizeof(uint32_t) * ((size_t)kBins + 4 * 256) * (size_t)wgs_per_row;
}
constexpr size_t ws_bytes_for(int slots, int wgs_per_row) {
  return kWsDataOff + (size_t)slots * slot_data_bytes(wgs_per_row);
}

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
  size_t slot_data_bytes;  // bytes per split-row data block
};

}  // namespace ert
