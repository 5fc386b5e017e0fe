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

// One-workgroup tier: the row's K output indices are staged in LDS and
// written with coalesced stores; the crossing bin's members (key, index)
// share that 16 KiB area, so their cap is (16 KiB - 4 K) / 8 members (1792,
// 1536, 1024 for K = 512, 1024, 2048).
constexpr int one_wg_cap(int k) { return (2 * kSingleCap * 4 - 4 * k) / 8; }

// The pages' rescue trigger is a crossing bin of more than
// min(CS x 4096, 32 x K, 16384) members with CS workgroups per row
// (PR 20998 "What changes").  Here the crossing-bin members of a row go
// through LDS for the refine in both tiers, so the trigger is m > kSingleCap.

// Launch variants: (workgroup size, float4 groups per thread).
struct Variant {
  int block;
  int qpt;
};
// One workgroup per row; resident capacity block * qpt * 4 scores.
// In order of capacity; the planner takes the first that holds the row.  Few
// waves per row keep the per-row fixed work (sample, scans, crossing, edges,
// refine) small next to the per-score work.
constexpr Variant kSingleVariants[] = {{256, 8}, {256, 17}, {512, 9}, {1024, 9}};
// G workgroups per row, each holding 1/G of the row; in order of capacity
// (the planner takes the first that holds a part).  The largest part runs
// 512 threads: a few long rows leave few workgroups per compute unit, and
// eight waves each hide more of a part's latency than four.
constexpr Variant kSplitVariants[] = {{256, 4}, {256, 8}, {512, 9}};
constexpr int kNumSplit = 3;

constexpr int kMaxWgsPerRow = 64;
constexpr int kMaxSlots = 256;  // split rows per launch (workspace slots)
constexpr int kStatsWords = 9;
constexpr int kBskMaxBlocks = 8192;  // rows the streaming pass takes: <= this many blocks of 32

// Workspace layout (bytes):
//   [0, 256)                             header (unused)
//   kMaxSlots fixed blocks of 17664 bytes: SlotHeader, digit counts [8][256],
//   value histogram [kBins]
//   then one data block per slot: G slices of kBins 16-bit suffix counts
//   (slice g: workgroup g's count of scores in bins >= b; a part holds fewer
//   than 2^16 scores), then the crossing bin's
//   members as (key, index) pairs [kSingleCap]
// The fixed blocks hold every word that carries state between workgroups, and
// the last workgroup of a row returns them all to zero; their place does not
// depend on the plan, so one workspace serves any plan it is large enough for.  Data blocks are written before they
// are read and need no clearing.
struct SlotHeader {
  uint32_t bar_count;  // barrier arrivals of the current row
  uint32_t done;       // workgroups finished with the slot (last one cleans)
  uint32_t win_cur;    // winner output cursor (rescue)
  uint32_t cand_cur;   // the row's maximum as an order-preserving key (retry)
  uint32_t tie_cur;    // tie tickets (rescue)
  // rescue: per radix level, the digit class's largest key and its smallest
  // key complemented, merged by atomic max (zero at rest); levels 0..3 of the
  // selection, then 0..3 of the deterministic tie pick
  uint32_t class_ext[16];
  uint32_t pad[43];    // header is 256 bytes
};
static_assert(sizeof(SlotHeader) == 256, "slot header size");

struct SlotFixed {
  SlotHeader hdr;
  uint32_t dig[8][256];  // rescue digit counts, one row per radix level
                         // (rows 4..7: the deterministic tie pick)
  uint32_t hist[2048];   // the row's value histogram (bins >= the floor bin)
  // Spacing only.  The slots' counters and histograms take atomics from every
  // workgroup of their rows; at a 16640-byte stride eight concurrent slots
  // measured about 15 % slower (memory-channel collisions), at 17664 not.
  uint32_t pad[256];
};
static_assert(sizeof(SlotFixed) == 17664, "slot fixed block size");

constexpr size_t kWsHeaderBytes = 256;
constexpr size_t kWsDataOff = kWsHeaderBytes + sizeof(SlotFixed) * kMaxSlots;
// Per-slot data block of a plan with G workgroups per row: G slices of
// kBins 16-bit suffix counts (one per workgroup), then the member list.
constexpr size_t kSliceBytes = sizeof(uint16_t) * kBins;
constexpr size_t kListBytes = 2 * sizeof(uint32_t) * kSingleCap;
constexpr size_t slot_data_bytes(int G) { return (size_t)G * kSliceBytes + kListBytes; }
constexpr size_t ws_bytes_for(int slots, int G) {
  return kWsDataOff + (size_t)slots * slot_data_bytes(G);
}

// The split tier's bounded row-barrier waits: the per-device count a wait
// that gives up adds to, and the polls a wait makes first.
struct BarrierSync {
  uint32_t* err = nullptr;
  uint32_t spins = 0;
};
constexpr uint32_t kDefaultSpins = 1u << 24;

// Fixed split-tier workspace of the entry point that allocates nothing: it
// holds every decode plan on a 256-compute-unit device (the largest needs
// about 22 MB); plans needing more are rejected.
constexpr size_t kScratchBytes = (size_t)24 << 20;

// Varlen / MTP decode form (the heuristic decode contract of PR 18122,
// run_varlen commit): row r belongs to request r / next_n, whose total cache
// length is kv_lens[r / next_n]; its window is [0, n) with
// n = (kv_len - next_n + r % next_n + 1) / compress_ratio, and no window when
// kv_len < next_n.
struct VarlenForm {
  const int32_t* kv_lens;  // per request, or nullptr
  int32_t next_n;
  int32_t compress_ratio;
};

struct GvrParams {
  const float* logits;
  int64_t row_stride;
  const int32_t* n_valid;     // decode form, or nullptr
  const int32_t* row_starts;  // prefill form
  const int32_t* row_ends;
  VarlenForm varlen;          // varlen decode form (kv_lens != nullptr)
  int32_t row_begin;  // first row handled by this launch
  int32_t rows;       // rows handled by this launch
  int32_t wgs_per_row;
  int32_t xcd_group;  // 1: map a row's workgroups onto one XCD
  int32_t cap;        // candidate cap of this plan
  int32_t force_rescue;
  int32_t deterministic;  // resolve the K-th value's tie class by smallest index
  const int32_t* hints;   // optional previous-step top-K positions (guess only)
  int64_t hint_stride;    // int32 entries between consecutive hint rows
  int32_t hint_div;       // row r reads hint row r / hint_div
  int32_t* indices;
  int32_t* row_stats;  // optional
  unsigned char* ws;   // workspace base (split tier), or nullptr
  BarrierSync sync;    // split tier: timeout count and poll limit
};

// Output epilogue (values, sorting): one workgroup per row.
constexpr int kEpiBlock = 256;

struct EpiParams {
  const float* logits;
  int64_t row_stride;
  const int32_t* n_valid;     // decode form, or nullptr
  const int32_t* row_starts;  // prefill form
  const int32_t* row_ends;
  VarlenForm varlen;
  int32_t row_begin;
  int32_t sorted;
  int32_t* indices;
  float* values;  // optional
};

}  // namespace ert
