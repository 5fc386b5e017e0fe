// gvr_kernels.hip -- gfx950 kernels of the exact per-row top-K
// (Guess-Verify-Refine with block64 sampling and an exact radix rescue).
//
// Steps per long row (nv > K), following the TensorRT-LLM page "GVR K=2048
// reg_clus with block64 sampling and parallel rescue" (PR 20998), sections
// "Why the GLM row overflows" and "What changes":
//  1. load the row once, as aligned float4 groups starting at col0 = ks & ~3
//     (PR 18702 "Kernel"); lanes outside [ks, ke) become NaN markers, never a
//     materialised -inf;
//  2. guess: K/64 blocks of 64 consecutive scores spread over the valid window
//     including both ends; the bracket is their min / max;
//  3. verify: histogram the row over kBins bins of the bracket (scores beyond
//     the bracket clamp into the end bins); an invalid bracket (non-finite or
//     collapsed) skips to the rescue;
//  4. the crossing bin b*: the highest bin whose count from the top reaches K;
//     everything above it is selected, b* holds m candidates of which
//     need = K - above are selected;
//  5. compact winners to the output and candidates to a buffer;
//  6. refine: the `need` largest candidates, exactly;
//  7. rescue when the bracket is invalid or the candidates overflow: an exact
//     4 x 8-bit radix select over the whole row's resident keys, using every
//     workgroup of the row, inside the same launch (it stops early on a digit
//     class that holds one key).
//
// Two tiers share the steps:
//  * one workgroup per row (SPLIT = false): the whole window is resident in
//    the workgroup's VGPRs, histogram, crossing bin, compaction and refine all
//    run in LDS, nothing is shared with other workgroups;
//  * G workgroups per row (SPLIT = true): each keeps 1/G of the row resident.
//    Every workgroup derives the same bracket and, from the sample's own
//    histogram, the same floor bin b_lo below which the crossing bin (almost
//    surely) is not.  Each counts its part's scores in bins >= b_lo in LDS
//    and adds those counts into the row's histogram in the workspace; after
//    one barrier every workgroup reads the merged counts and finds the same
//    crossing bin; the suffix counts the workgroups published give each its
//    offsets.  It appends its crossing-bin members to a short list, counts
//    itself done, then writes its winners straight to the output; the last
//    workgroup to finish refines that list.  A row whose merged counts do
//    not reach K (the floor was too high), whose crossing bin is crowded, or
//    whose bracket is invalid takes the parallel rescue with all its
//    workgroups, the radix levels merging through the workspace behind the
//    same kind of barrier.
//
// Ordering: scores compare as IEEE values with -0 == +0; the order-preserving
// key maps a float to a uint32 whose unsigned order is that value order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gvr_common.h"
#include "gvr_device.h"
#include "row_window.h"

namespace ert {

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <int K, int BLOCK>
struct alignas(16) Smem {
  union {
    uint32_t hist[kBins + 64];  // + one trash word per lane for NaN markers
    struct {                    // split tier: the row's member list (last workgroup)
      uint32_t key[kSingleCap];
      int32_t idx[kSingleCap];
    } c;
    struct {                    // one-workgroup tier: the staged output row and the
      int32_t ob[K];            // crossing bin's members
      uint32_t key[one_wg_cap(K)];
      int32_t idx[one_wg_cap(K)];
    } o;
  } u;
  alignas(16) uint32_t dh[256];  // radix digit counts (cleared as 16-byte words)
  uint32_t mm[2 * (BLOCK / 64)];  // per-wave class extremes of a radix level
  uint32_t scan[BLOCK / 64];
  float rmin[BLOCK / 64];
  float rmax[BLOCK / 64];
  float hmin[BLOCK / 64];
  float hmax[BLOCK / 64];
  Cross cross;
  float thr[2];
  uint32_t bc[4];
  uint32_t ctr[4];
};

// Occupancy targets of the one-workgroup variants (waves per SIMD; the VGPR
// budget is 512 / waves, in granules of 8):
//  * up to 9 groups per thread and 256 threads, or 512 threads for K <= 1024:
//    8 (64 VGPRs), so that four 512-thread workgroups share a compute unit
//    (512 threads at K = 2048 would spill there);
//  * 256 threads and 17 groups: 5 (96 VGPRs; one more granule would drop a
//    wave per SIMD, about 10 % of a full-chip pass).
// The split variants and the 1024-thread one keep the compiler's choice.
template <int K, int QPT, int BLOCK, bool SPLIT>
struct WavesPerEu {
  static constexpr int value = SPLIT                          ? 1
                               : (QPT <= 9 && (BLOCK == 256 || (BLOCK == 512 && K <= 1024))) ? 8
                               : (BLOCK == 256 && QPT == 17)  ? 5
                                                              : 1;
};

// ---------------------------------------------------------------------------
// One row in two halves: row_begin resolves the row and issues its loads
// (the sample, then the part into v), row_finish selects.  The state the
// loads leave for the selection travels in a RowCtx (uniform values).
// ---------------------------------------------------------------------------

template <int K, int BLOCK>
constexpr int spw() {  // sample blocks per wave
  return (K / 64 + BLOCK / 64 - 1) / (BLOCK / 64);
}

struct RowCtx {
  int nv, lead, span, Q, q0, q1, qw0, nj, jf0, jf1;
  int32_t* out;
  int32_t* stats;
  SlotFixed* sf;
  SlotHeader* hdr;
  uint16_t* slices;
  uint2* s_pair;
  const int32_t* hrow;
};

// Resolves row `slot` (part g) and issues its loads; false when the row is
// finished already (a short row: identity written).  Split-tier hints write
// the workgroup's LDS; the one-workgroup tier's loads touch no LDS.
template <int K, int QPT, int BLOCK, bool SPLIT>
__device__ __forceinline__ bool row_begin(const GvrParams& p, Smem<K, BLOCK>& sm, int slot, int g,
                                          RowCtx& c, f4 (&v)[QPT],
                                          float (&smp)[spw<K, BLOCK>()]) {
  constexpr int W = BLOCK / 64;           // waves
  constexpr int NSB = K / 64;             // sample blocks
  constexpr int SPW = (NSB + W - 1) / W;  // sample blocks per wave
  const int t = threadIdx.x;
  const int G = SPLIT ? p.wgs_per_row : 1;
  const int64_t row = (int64_t)p.row_begin + slot;

  // ---- row resolve (a0); row_stride < 2^30 is checked on the host --------
  const int S = (int)p.row_stride;
  int ks, nv;
  row_window(p.n_valid, p.row_starts, p.row_ends, p.varlen, row, S, &ks, &nv);
  int32_t* out = p.indices + row * K;
  int32_t* stats = p.row_stats ? p.row_stats + row * kStatsWords : nullptr;

  // ---- short row (a1): identity then -1 ----------------------------------
  if (nv <= K) {
    for (int i = g * BLOCK + t; i < K; i += G * BLOCK) store_nt(out + i, (i < nv) ? i : -1);
    if (stats && g == 0 && t < kStatsWords)
      stats[t] = (t == 0) ? 0 : (t == 6 ? G : (t == 7 ? p.cap : -1));
    return false;
  }

  // ---- part of the row this workgroup owns -------------------------------
  const int col0 = ks & ~3;
  const int lead = ks & 3;
  const int span = lead + nv;     // positions [0, span) from col0
  const int Q = (span + 3) >> 2;  // float4 groups
  int q0 = 0, q1 = Q;
  if (SPLIT) {
    const int Qp = (Q + G - 1) / G;
    q0 = g * Qp;
    q1 = q0 + Qp < Q ? q0 + Qp : Q;
  }
  const float* rowp = p.logits + row * (int64_t)S;
  const f4* base = reinterpret_cast<const f4*>(rowp + col0);

  SlotFixed* sf = nullptr;
  SlotHeader* hdr = nullptr;
  uint16_t* slices = nullptr;  // per-workgroup 16-bit suffix counts [G][kBins]
  uint2* s_pair = nullptr;     // crossing-bin members (key, index)
  if (SPLIT) {
    sf = reinterpret_cast<SlotFixed*>(p.ws + kWsHeaderBytes) + slot;
    hdr = &sf->hdr;
    unsigned char* data = p.ws + kWsDataOff + (size_t)slot * slot_data_bytes(G);
    slices = reinterpret_cast<uint16_t*>(data);
    s_pair = reinterpret_cast<uint2*>(data + (size_t)G * kSliceBytes);
  }

  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, uniform
  const int l = lane_id();
  const float qnan = __builtin_nanf("");

  // ---- guess (a3): block64 sample over the valid window -------------------
  // Block j starts at floor(j * (nv - 64) / (NSB - 1)); blocks are disjoint
  // for nv > K, so the sample holds exactly K distinct scores, and the first
  // and last blocks touch both ends of the window.  Wave w reads blocks
  // w, w + W, ...: one 256-byte load per block.
  {
    const float* win = rowp + ks;
    const SampleStep<NSB> ss(nv);
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int j = w + i * W;
      if (j < NSB) {
        const int st = ss.start(j);
        smp[i] = win[st + l];
      } else {
        smp[i] = qnan;
      }
    }
  }

  // ---- hint-guided guess (a3 variant): positions ---------------------------
  // Optional: the caller's hint positions -- the previous decode step's top-K
  // of the same request, raw, possibly stale or degenerate.  They only steer
  // the bracket; every later step is exact whatever they hold.  Each thread
  // takes one hint slot (the first min(K, BLOCK) slots): one gather per
  // thread instead of K / BLOCK keeps the dependent, line-per-lane loads
  // cheap, and the extremes over a few hundred hint scores already sit near
  // those of the whole hint set.  The split tier reads them up front: its
  // positions first, so that the scores are gathered before the part's loads
  // are issued and the bracket overlaps the part's flight as it does without
  // hints.  A one-workgroup row does not read them: when its first bracket
  // fails it retries with the row's own maximum, which it holds (below).
  const int32_t* hrow = nullptr;
  if (p.hints) {
    // rows and hint_div are positive int32: a 32-bit unsigned divide
    const uint32_t req = (uint32_t)row / (uint32_t)p.hint_div;
    hrow = p.hints + (int64_t)req * p.hint_stride;
  }
  int32_t hpos = -1;
  if (SPLIT && hrow && t < K) hpos = hrow[t];

  // ---- hint-guided guess: scores -------------------------------------------
  // A hint outside [0, nv) (the -1 pad of a short row, a position past the
  // window) is skipped by an unsigned compare; a NaN leaves min / max as is.
  if (SPLIT && hrow) {
    float x = qnan;
    if ((uint32_t)hpos < (uint32_t)nv) x = rowp[ks + hpos];
    float hlo = x, hhi = x;
    wave_minmax(hlo, hhi);
    if (l == 0) {
      sm.hmin[w] = hlo;
      sm.hmax[w] = hhi;
    }
    // keep the part's loads behind this point: issued earlier, they would
    // hold their registers while the gather waits (loads complete in order)
    asm volatile("" ::: "memory");
  }

  // ---- scan (a2): the part, resident in VGPRs -----------------------------
  // Thread t holds groups q0 + t + j * BLOCK, j < QPT: each load instruction
  // of a wave reads 1 KiB of consecutive scores.  Lanes outside the window or
  // the part (the <= 3 lead lanes, the tail of the last group, groups past the
  // part) become NaN markers here: no selection step accepts a NaN (its
  // compares are false, its histogram increment goes to a trash word, its
  // rescue key is the lowest key), and a genuine -inf tie class stays intact.
  // Per-wave group counts (uniform, computed once): this wave holds groups
  // j < nj (those starting before the part's end q1), and groups
  // jf0 <= j < jf1 hold four in-window scores in all 64 lanes ("full": the
  // passes skip their marker checks).  Every pass compares its unrolled j
  // with these counts, so no per-group flags stay live across passes.
  const int qw0 = __builtin_amdgcn_readfirstlane(q0 + w * 64);
  const int qf1 = min(q1, span >> 2);  // groups wholly inside the window and the part
  const int nj = __builtin_amdgcn_readfirstlane(qw0 < q1 ? min((q1 - qw0 + BLOCK - 1) / BLOCK, QPT) : 0);
  const int jf0 = __builtin_amdgcn_readfirstlane((qw0 == 0 && lead > 0) ? 1 : 0);
  const int jf1 = __builtin_amdgcn_readfirstlane(
      qw0 + 64 <= qf1 ? min((qf1 - qw0 - 64) / BLOCK + 1, QPT) : 0);
  // Buffer loads whose range ends at the part's end: lanes past it (only in
  // the wave holding the part's last group) read zeros without a memory
  // access and become markers below.  The whole offset sits in the per-lane
  // offset, which the range check covers.
  // Every one of the QPT loads is issued, also past the part's end (those
  // read zeros without a memory access and no pass looks at them): with a
  // fixed count of loads behind the sample's, the waits for the sample (and
  // for a group) are exact counts, so the bracket and, in the split tier,
  // the sample's floor run while the part is still in flight.
  {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, q1 * 16);
    const int vo = (qw0 + l) * 16;
#pragma unroll
    for (int j = 0; j < QPT; ++j)
      v[j] = __builtin_bit_cast(
          f4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, vo + j * BLOCK * 16, 0, kCachePolicyNT));
  }
  c.nv = nv;
  c.lead = lead;
  c.span = span;
  c.Q = Q;
  c.q0 = q0;
  c.q1 = q1;
  c.qw0 = qw0;
  c.nj = nj;
  c.jf0 = jf0;
  c.jf1 = jf1;
  c.out = out;
  c.stats = stats;
  c.sf = sf;
  c.hdr = hdr;
  c.slices = slices;
  c.s_pair = s_pair;
  c.hrow = hrow;
  return true;
}

// The selection of a row whose loads row_begin issued.
template <int K, int QPT, int BLOCK, bool SPLIT>
__device__ __forceinline__ void row_finish(const GvrParams& p, Smem<K, BLOCK>& sm, int g,
                                           const RowCtx& c, f4 (&v)[QPT],
                                           float (&smp)[spw<K, BLOCK>()]) {
  constexpr int W = BLOCK / 64;           // waves
  constexpr int NSB = K / 64;             // sample blocks
  constexpr int SPW = (NSB + W - 1) / W;  // sample blocks per wave
  constexpr int NW = (QPT * 4 + 31) / 32;
  const int t = threadIdx.x;
  const int G = SPLIT ? p.wgs_per_row : 1;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, uniform
  const int l = lane_id();
  const float qnan = __builtin_nanf("");
  const int nv = c.nv, lead = c.lead, span = c.span, Q = c.Q, q0 = c.q0, q1 = c.q1;
  const int qw0 = c.qw0, nj = c.nj, jf0 = c.jf0, jf1 = c.jf1;
  int32_t* const out = c.out;
  int32_t* const stats = c.stats;
  SlotFixed* const sf = c.sf;
  SlotHeader* const hdr = c.hdr;
  uint16_t* const slices = c.slices;
  uint2* const s_pair = c.s_pair;
  const int32_t* const hrow = c.hrow;
  (void)NSB;
  (void)slices;
  (void)s_pair;
  // Visit this thread's groups; `full` (uniform per wave) says all 64 lanes
  // hold four in-window scores, so only boundary waves pay for NaN checks.
  auto each = [&](auto&& f) {
    // Opaque copies of the lane index and the counts: every pass recomputes
    // its group indices and tests instead of the compiler keeping one set
    // live across all passes.
    int ll = l, njp = nj, jf0p = jf0, jf1p = jf1;
    asm volatile("" : "+v"(ll));
    asm volatile("" : "+s"(njp));
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      if (j < njp) {
        const int q = qw0 + j * BLOCK + ll;
        const bool full = j >= jf0p && j < jf1p;
        f(j, q, full);
      }
    }
  };
  auto resident = [&](auto&& f) {
    each([&](int j, int q, bool) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // opaque copy: the key is recomputed per radix level, not kept live
        float x = v[j][e];
        asm volatile("" : "+v"(x));
        f(rkey(x));
      }
    });
  };

  // ---- bracket -------------------------------------------------------------
  float smin = smp[0], smax = smp[0];
#pragma unroll
  for (int i = 1; i < SPW; ++i) {
    smin = fminf(smin, smp[i]);
    smax = fmaxf(smax, smp[i]);
  }
  wave_minmax(smin, smax);
  if (l == 0) {
    sm.rmin[w] = smin;
    sm.rmax[w] = smax;
  }
  for (int i = t; i < (kBins + 64) / 4; i += BLOCK)
    reinterpret_cast<uint4*>(sm.u.hist)[i] = uint4{0u, 0u, 0u, 0u};
  if (t < 4) {
    sm.ctr[t] = 0u;
    sm.bc[t] = 0u;
  }
  lds_sync();
  float gmin = sm.rmin[0], gmax = sm.rmax[0];
#pragma unroll
  for (int i = 1; i < W; ++i) {
    gmin = fminf(gmin, sm.rmin[i]);
    gmax = fmaxf(gmax, sm.rmax[i]);
  }
  // uniform: scalar registers, out of the resident row's VGPR budget
  gmin = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gmin)));
  gmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gmax)));
  // Usable hints (finite, at least two distinct scores) raise the bracket's
  // top to the highest hint score when it lies above the sample's maximum:
  // peaks the sample missed then get bins of their own instead of piling up
  // in the top bin.  The split tier also lets the lowest hint score lower its
  // floor (below).  Degenerate hints (all one position, all invalid, all -1)
  // change nothing.
  // (the per-wave extremes in sm.hmin / sm.hmax, reduced over the workgroup)
  auto hint_extremes = [&](float& hl, float& hh) {
    hl = sm.hmin[0];
    hh = sm.hmax[0];
#pragma unroll
    for (int i = 1; i < W; ++i) {
      hl = fminf(hl, sm.hmin[i]);
      hh = fmaxf(hh, sm.hmax[i]);
    }
    // every lane read the same words: keep them in scalar registers
    hl = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(hl)));
    hh = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(hh)));
  };
  bool hint_ok = false;
  float hfloor = 0.0f;
  if (SPLIT && hrow) {
    float hl, hh;
    hint_extremes(hl, hh);
    if (__builtin_isfinite(hl) && __builtin_isfinite(hh) && hh > hl) {
      hint_ok = true;
      hfloor = hl;
      gmax = fmaxf(gmax, hh);
    }
  }
  BinMap bm;
  const bool bracket_ok = bm.set(gmin, gmax) && !p.force_rescue;

  // The lead / tail lanes become NaN markers only after the bracket (and in
  // the split tier after the sample's floor), so that work does not wait
  // for the whole part to arrive.
  auto mark_ends = [&]() {
    // first group of the window (lead lanes): q == 0 is thread 0's j == 0
    if (q0 == 0 && t == 0 && lead > 0) {
#pragma unroll
      for (int e = 0; e < 3; ++e)
        if (e < lead) v[0][e] = qnan;
    }
    // last group of the part: the lanes after it in its wave hold a copy of
    // it; in the window's last group the scores past the tail go too
    if (q1 > q0) {
      // group jl (uniform) of thread tl holds it: only that thread's wave
      // takes the branch, and only group jl's registers are touched
      const int d = q1 - 1 - q0;
      const int jl = d / BLOCK;
      const int tl = d - jl * BLOCK;
      const int lt = tl & 63;
      const int tail = q1 == Q ? span - ((Q - 1) << 2) : 4;  // scores of the last group, 1..4
      if (w == (tl >> 6) && (lt < 63 || tail < 4)) {
        if constexpr (QPT <= 4) {
          // (selects on every group: with so few groups the compiler turns
          // the branch form below into one store at a computed index, which
          // moves the row's registers to scratch memory)
#pragma unroll
          for (int j = 0; j < QPT; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool keep = j != jl || l < lt || (l == lt && e < tail);
              v[j][e] = keep ? v[j][e] : qnan;
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < QPT; ++j)
            if (j == jl) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool keep = l < lt || (l == lt && e < tail);
                v[j][e] = keep ? v[j][e] : qnan;
              }
            }
        }
      }
    }
  };

  int floor_bin = -1;  // split tier: the floor bin its histogram counts from
  auto put_stats = [&](int path, int m, int above, int b) {
    if (stats && t == 0) {
      stats[0] = path;
      stats[1] = m;
      stats[2] = above;
      stats[3] = b;
      stats[4] = (int)__float_as_uint(gmin);
      stats[5] = (int)__float_as_uint(gmax);
      stats[6] = G;
      stats[7] = p.cap;
      stats[8] = floor_bin;
    }
  };

  uint32_t nbar = 0;  // row barriers this workgroup has passed (split tier)
  int path = 2;  // 1 fast, 2 rescue (invalid bracket), 3 rescue (crowded top)
  Cross cr{-1, 0u, 0u, 0u};

  float xf = -__builtin_inff();  // one-workgroup retry: the counted scores' floor
  if (!SPLIT) mark_ends();
  if (!SPLIT) {
    // ==== one workgroup per row ============================================
    if (bracket_ok) {
      // ---- verify (a4, a5): LDS histogram and crossing bin ---------------
      // (masked: only scores >= xf are counted -- the retry below)
      auto verify = [&](const bool masked) {
        if (masked) {
          each([&](int j, int q, bool) {
            int b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = v[j][e];
              b[e] = x >= xf ? (int)vbin_off(x, bm) : -1;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (b[e] >= 0) lds_inc(hword(sm.u.hist, (uint32_t)b[e]));
          });
        } else {
          // Every visited score is counted, the NaN markers with the rest:
          // they all land in the one bin a NaN maps to, and each wave takes
          // its markers out of it below (no per-group test, no per-score
          // NaN check).
          each([&](int j, int q, bool) {
#pragma unroll
            for (int e = 0; e < 4; ++e) lds_inc(hword(sm.u.hist, vbin_off(v[j][e], bm)));
          });
          // The wave's markers: its visited groups hold 256 scores each
          // (window positions 4 qw0 + 1024 j - lead onwards); only the first
          // (the window's lead) and the last (the window's end) can reach
          // outside [0, nv).
          int njp = nj;
          asm volatile("" : "+s"(njp));
          if (l == 0 && njp > 0) {
            auto inwin = [&](int j) {  // in-window scores of the wave's group j
              const int st = 4 * (qw0 + j * BLOCK) - lead;
              const int lo = st > 0 ? st : 0;
              const int hi = st + 256 < nv ? st + 256 : nv;
              return hi > lo ? hi - lo : 0;
            };
            const int inside = njp == 1 ? inwin(0) : inwin(0) + 256 * (njp - 2) + inwin(njp - 1);
            const uint32_t mk = (uint32_t)(256 * njp - inside);
            if (mk) (void)__hip_atomic_fetch_sub(hword(sm.u.hist, vbin_off(qnan, bm)), mk,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
        lds_sync();
        cr = crossing_1sync<BLOCK>(sm.u.hist, (uint32_t)K, sm.scan);
        path = (cr.b >= 0 && cr.m <= (uint32_t)one_wg_cap(K)) ? 1 : 3;
      };
      verify(false);
      if (path == 3 && cr.b == kBins - 1) {
        // The crossing bin is the top one, over the cap: scores above the
        // sample's maximum (peaks the sample missed) pile up there.  Count
        // again over [that bin's lower edge, the row's own maximum], only
        // the scores at or above the edge (a crowd at the maximum itself
        // still takes the rescue).
        float mx = -__builtin_inff();
        each([&](int j, int q, bool) {
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, v[j][e]);  // NaN markers drop out
        });
        float mn = mx;
        wave_minmax(mn, mx);
        if (l == 0) sm.hmax[w] = mx;
        if (w == 0) {
          const float e = bin_edge(kBins - 1, bm);
          if (l == 0) sm.thr[0] = e;
        }
        lds_sync();
        float top = sm.hmax[0];
#pragma unroll
        for (int i = 1; i < W; ++i) top = fmaxf(top, sm.hmax[i]);
        top = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(top)));
        const float lo = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.thr[0])));
        BinMap rm;
        if (rm.set(lo, top)) {
          gmin = lo;
          gmax = top;
          bm = rm;
          xf = lo;
          for (int i = t; i < kBins + 64; i += BLOCK) sm.u.hist[i] = 0u;
          lds_sync();
          verify(true);
          if (path == 1) path = 5;
        }
      }
    }
    if (path == 1 || path == 5) {
      // ---- compaction (a6) ------------------------------------------------
      // bin > b*  <=>  x >= x_hi (winner);  bin == b*  <=>  x_lo <= x < x_hi
      // (after the retry bin 0 also holds what lies below its floor xf)
      if (w < 2) {
        // (the upper edge of the top bin is NaN, which no score reaches: no
        // clamp there)
        const float e = bin_edge(cr.b + w, bm);
        if (l == 0) sm.thr[w] = w == 0 ? fmaxf(e, xf) : e;
      }
      lds_sync();
      const uint32_t need = (uint32_t)K - cr.above;
      uint32_t wb[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) wb[i] = 0u;
      // this thread's winner bits (x >= x_hi), shifted in group by group;
      // members (x_lo <= x < x_hi) go to the LDS list as they are met
      int ngrp = 0;  // groups this wave visited (uniform)
      {
        const float xlo = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.thr[0])));
        const float xhi = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.thr[1])));
        each([&](int j, int q, bool) {
          uint64_t gm[4];
          group_wins(v[j], xlo, xhi, wb[j >> 3], gm);
          if ((gm[0] | gm[1] | gm[2] | gm[3]) != 0ull)
            append_members(v[j], (q << 2) - lead, gm, &sm.bc[0], sm.u.o.key, sm.u.o.idx,
                           (uint32_t)one_wg_cap(K));
          ngrp = j + 1;
        });
      }
      uint32_t nwin = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) nwin += __popc(wb[i]);
      const uint32_t ex = wave_offsets(nwin, &sm.bc[0]);
      // word d holds groups 8d .. 8d + 7, nd bits shifted in: bit p is this
      // thread's score i = 32 d + nd - 1 - p (group i / 4, lane i % 4)
      auto nbits = [&](int d) { return 4 * min(max(ngrp - 8 * d, 0), 8); };
      {
        // (staged in LDS: stored straight from the walk, each winner was its
        // own scattered 4-byte write, and on the prefill tile those writes
        // kept the compute units' address units busy while the rows' loads
        // queued behind them)
        // The slots need no bound: every winner lies in a bin above the
        // crossing one (the edge is exact), so the winners number at most
        // cr.above <= K.
        uint32_t wo = (ex & 0xFFFFu) * 4u;  // byte offset of the next slot
        const int base = ((q0 + t) << 2) - lead;
#pragma unroll
        for (int d = 0; d < NW; ++d) {
          const int nb = nbits(d);  // uniform
          if (nb == 0) break;
          uint32_t bits = wb[d] << (32 - nb);
          const int bd = base + 32 * d * BLOCK;
          while (bits) {
            const uint32_t c = walk_pop(bits);
            *reinterpret_cast<int32_t*>(reinterpret_cast<char*>(sm.u.o.ob) + wo) =
                bd + walk_offset<BLOCK>(c);
            wo += 4u;
            asm volatile("" : "+v"(wo));
          }
        }
      }
      lds_sync();
      // ---- output (a9) and refine (a7) ------------------------------------
      // The winners staged by the walk go out with coalesced stores, and the
      // refine writes its `need` picks straight to the output: no barrier
      // follows, so no wave waits for these stores (a barrier waits for the
      // wave's outstanding stores) or for another wave's refine.
      const uint32_t m = cr.m;
      int32_t* const ob = sm.u.o.ob;
      auto put_rows = [&](uint32_t b0, uint32_t b1) {  // ob[b0, b1) -> out, b0 % 4 == 0
        if ((reinterpret_cast<uintptr_t>(out) & 15u) == 0u) {
          const uint32_t e4 = b1 & ~3u;
          for (uint32_t i = b0 + 4u * t; i < e4; i += 4u * BLOCK) store_nt4(out + i, ob + i);
          if ((uint32_t)t < b1 - e4) store_nt(out + e4 + t, ob[e4 + t]);
        } else {
          for (uint32_t i = b0 + t; i < b1; i += BLOCK) store_nt(out + i, ob[i]);
        }
      };
      if (need == m || m <= (uint32_t)kRankMax) {
        put_rows(0u, cr.above);
        if (need == m) {
          for (uint32_t i = t; i < m; i += BLOCK) store_nt(out + cr.above + i, sm.u.o.idx[i]);
        } else {
          rank_select_direct<BLOCK>(sm.u.o.key, sm.u.o.idx, m, need, out, cr.above);
        }
      } else {
        list_select<BLOCK>(sm.u.o.key, sm.u.o.idx, m, need, p.deterministic != 0, ob, cr.above,
                           (uint32_t)K, sm.dh, &sm.cross, sm.scan, sm.mm, sm.ctr, nbar);
        lds_sync();
        put_rows(0u, (uint32_t)K);
      }
      put_stats(path, (int)cr.m, (int)cr.above, cr.b);
      return;
    }
  } else {
    // ==== G workgroups per row =============================================
    int blo = 0;
    if (bracket_ok) {
      // Floor bin from the sample alone: the sample holds about
      // lam = K*K/nv scores >= the row's K-th value, so the bin where the
      // sample's count from the top reaches lam plus a wide margin lies at
      // or below the crossing bin (almost surely; a row where it does not is
      // caught below and finished exactly all the same).
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const float x = smp[i];
        lds_inc(hword(sm.u.hist, (x == x) ? vbin_off(x, bm) : 4u * (uint32_t)(kBins + l)));
      }
      lds_sync();
      const float lam = (float)K * (float)K / (float)nv;
      const float rl = lam + 4.0f * sqrtf(lam) + 8.0f;
      const uint32_t rlow = rl >= (float)K ? (uint32_t)K : (uint32_t)rl;
      const Cross sc0 = crossing_1sync<BLOCK>(sm.u.hist, rlow, sm.scan);
      blo = sc0.b > 0 ? sc0.b : 0;
      if (hint_ok) {
        // Hint-guided floor: the previous step's top-K mostly stays above
        // this step's K-th value, so a sample floor above the lowest hint
        // score is suspect (the sample may have met a dense cluster the rest
        // of the row does not share).  Lower the floor to the hint's bin,
        // unless the hint sits far below where the sample puts the K-th
        // value (stale hints at the row's bottom would only add work):
        // the sample's count must not pass lam + 8 sqrt(lam) + 16 above it.
        const int bh = vbin(hfloor, bm);
        if (bh < blo) {
          const float ru = lam + 8.0f * sqrtf(lam) + 16.0f;
          int bup = -1;
          if (ru < (float)K) bup = crossing_1sync<BLOCK>(sm.u.hist, (uint32_t)ru, sm.scan).b;
          if (bh >= bup) blo = bh;
        }
      }
      floor_bin = blo;
      // A sample bin at or above the floor holding 8 or more samples marks a
      // row with heavy ties there: its histogram pass aggregates per wave.
      // One holding so many that its scores (each sample stands for nv / K
      // of them) would fill the member list twice over predicts a crossing
      // bin over the cap: such a bin cannot lie above the crossing (it holds
      // more than K scores) nor between the floor and it (the floor's count
      // would pass lam + margin there), so the row goes straight to the
      // rescue instead of paying for the fast path first.  At least 32
      // samples, half a sample block: a few neighbouring scores of one block
      // can share a bin on a smooth stretch of the row without the row being
      // crowded.
      const float crowded = fmaxf(2.0f * (float)kSingleCap * (float)K / (float)nv, 32.0f);
      lds_sync();  // every wave has read the sample's counts
      {
        // four bins per read; each thread then clears what it read
        uint32_t mx = 0u;
        for (int i4 = t; i4 < (kBins + 64) / 4; i4 += BLOCK) {
          uint4* p4 = reinterpret_cast<uint4*>(sm.u.hist) + i4;
          if (i4 < kBins / 4) {
            const uint4 c = *p4;
            const int b = 4 * i4;
            mx = max(mx, b >= blo ? c.x : 0u);
            mx = max(mx, b + 1 >= blo ? c.y : 0u);
            mx = max(mx, b + 2 >= blo ? c.z : 0u);
            mx = max(mx, b + 3 >= blo ? c.w : 0u);
          }
          *p4 = uint4{0u, 0u, 0u, 0u};
        }
        if (mx >= 8u) sm.bc[3] = 1u;
        if ((float)mx >= crowded) sm.ctr[3] = 1u;
      }
      lds_sync();
      path = sm.ctr[3] ? 3 : 1;
    }
    mark_ends();
    // One verify round: the part's scores >= edge(bl) counted per bin in
    // LDS, merged into gh (zero on entry) through the workspace behind a row
    // barrier, the crossing bin -> cr.  Returns the path: 1 fast, 3 crowded
    // crossing bin, 4 merged counts short of K (the floor lay above the K-th
    // value).
    float xfloor = -__builtin_inff();  // a retry's explicit floor value
    auto verify = [&](const int bl, uint32_t* gh) -> int {
      // ---- verify (a4): the row's histogram on bins >= blo ----------------
      // Each workgroup counts its part's scores >= edge(blo) per bin in LDS,
      // adds the non-zero counts into the row's histogram in the workspace
      // and publishes its suffix counts (its scores in bins >= b, for each
      // b >= blo) in its slice.  After one barrier every workgroup reads the
      // row's histogram and finds the same crossing bin; the slices of the
      // workgroups before it say where its winners and members go.  Bins
      // below blo are not needed: were the crossing bin there, the merged
      // counts would not reach K and the row would take the rescue.
      if (w == 0) {
        const float e = bin_edge(bl, bm);
        if (l == 0) sm.thr[0] = e;
      }
      lds_sync();
      const float xf = fmaxf(sm.thr[0], xfloor);
      if (sm.bc[3]) {
        each([&](int j, int q, bool) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = v[j][e];
            const bool in = x >= xf;
            lds_inc_agg(sm.u.hist, in ? (uint32_t)vbin(x, bm) : 0u, in);
          }
        });
      } else {
        // only the lanes whose score reaches the floor take part in each
        // increment: the LDS cost follows the active lanes
        each([&](int j, int q, bool) {
          int b[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = v[j][e];
            b[e] = x >= xf ? (int)vbin_off(x, bm) : -1;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (b[e] >= 0) lds_inc(hword(sm.u.hist, (uint32_t)b[e]));
        });
      }
      lds_sync();
      {
        // suffix counts: thread t owns PER consecutive bins from the top and
        // writes them as 16-bit counts, four to an 8-byte word (whole lines
        // per wave), with the agent-coherent cache policy; groups wholly
        // below the floor are skipped (nothing reads a slice below the
        // crossing bin)
        static_assert(BLOCK * QPT * 4 < 65536, "a part's counts fit 16 bits");
        constexpr int PER = kBins / BLOCK;
        const int hi = kBins - 1 - t * PER;
        uint32_t c[PER];
        uint32_t sum = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          c[i] = hi - i >= bl ? sm.u.hist[hi - i] : 0u;
          sum += c[i];
        }
        uint32_t tot;
        uint32_t run = block_excl_scan<BLOCK>(sum, sm.scan, tot);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(slices + (size_t)g * kBins, kBins * 2);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          run += c[i];
          c[i] = run;
        }
        if constexpr (PER % 4 == 0) {
#pragma unroll
          for (int q4 = 0; q4 < PER / 4; ++q4) {
            const int b0 = hi - PER + 1 + 4 * q4;  // the group's lowest bin
            if (b0 + 3 >= bl) {
              typedef uint32_t v2u __attribute__((ext_vector_type(2)));
              const v2u sv = {c[PER - 1 - 4 * q4] | (c[PER - 2 - 4 * q4] << 16),
                              c[PER - 3 - 4 * q4] | (c[PER - 4 - 4 * q4] << 16)};
              __builtin_amdgcn_raw_buffer_store_b64(sv, rs, b0 * 2, 0, kCachePolicyAgent);
            }
          }
        } else {
          // (no split part runs more than 512 threads)
          uint16_t* mine = slices + (size_t)g * kBins;
#pragma unroll
          for (int i = 0; i < PER; ++i)
            if (hi - i >= bl)
              __hip_atomic_store(&mine[hi - i], (uint16_t)c[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // the row's histogram: one bin per lane, consecutive across a wave
        for (int b = t; b < kBins; b += BLOCK) {
          const uint32_t n = b >= bl ? sm.u.hist[b] : 0u;
          if (n) atomic_add_agent_nr(&gh[b], n);
        }
      }
      row_barrier(hdr, G, nbar, p.sync);
      {
        constexpr int BPT = kBins / BLOCK;
        uint32_t r[BPT];
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          const int b = t + i * BLOCK;
          r[i] = b >= bl ? load_agent(&gh[b]) : 0u;
        }
#pragma unroll
        for (int i = 0; i < BPT; ++i) sm.u.hist[t + i * BLOCK] = r[i];
      }
      lds_sync();
      // ---- crossing bin (a5), the same in every workgroup of the row -----
      cr = crossing_1sync<BLOCK>(sm.u.hist, (uint32_t)K, sm.scan);
      // Merged counts below K (the sample's floor lay above the K-th value)
      // or a crowded crossing bin: the row's workgroups take the rescue
      // together.
      return cr.b < 0 ? 4 : (cr.m > (uint32_t)kSingleCap ? 3 : 1);
    };
    if (path == 1) {
      path = verify(blo, sf->hist);
      // Two failures get a second counting round, merged into the digit rows
      // (zero at rest), rather than the radix rescue:
      //  * merged counts short of K: the floor lay above the K-th value (a
      //    sample that met a stretch of high scores the rest of the row does
      //    not share) -- count again with no floor;
      //  * the crossing bin is the top one, over the cap: scores above the
      //    sample's maximum (peaks the sample missed) piled up there -- count
      //    again over [that bin's lower edge, the row's maximum], only the
      //    scores at or above the edge.  The row's maximum is merged through
      //    the slot header (an atomic max of order-preserving keys).
      bool retry = path == 4;
      if (path == 3 && cr.b == kBins - 1) {
        float mx = -__builtin_inff();
        each([&](int j, int q, bool) {
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, v[j][e]);  // NaN markers drop out
        });
        float mn = mx;
        wave_minmax(mn, mx);
        if (l == 0) sm.hmax[w] = mx;
        if (w == 0) {
          const float e = bin_edge(kBins - 1, bm);
          if (l == 0) sm.thr[0] = e;
        }
        lds_sync();
        if (t == 0) {
          float pm = sm.hmax[0];
          for (int i = 1; i < W; ++i) pm = fmaxf(pm, sm.hmax[i]);
          if (pm == pm && pm > -__builtin_inff())
            __hip_atomic_fetch_max(&hdr->cand_cur, fkey(pm), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        const float lo = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.thr[0])));
        row_barrier(hdr, G, nbar, p.sync);
        const uint32_t tk = __builtin_amdgcn_readfirstlane(load_agent(&hdr->cand_cur));
        const float top = tk ? from_key(tk) : -__builtin_inff();
        BinMap rm;
        if (rm.set(lo, top)) {
          gmin = lo;
          gmax = top;
          bm = rm;
          xfloor = lo;
          retry = true;
        }
      }
      if (retry) {
        lds_sync();  // every wave has read the merged counts
        for (int i = t; i < kBins + 64; i += BLOCK) sm.u.hist[i] = 0u;
        floor_bin = 0;
        path = verify(0, &sf->dig[0][0]);
        if (path == 1) {
          path = 5;
        } else {
          // the rescue merges its digit counts in those rows: every
          // workgroup has read them; back to zero, then on
          row_barrier(hdr, G, nbar, p.sync);
          for (int i = t; i < 8 * 256; i += BLOCK)
            __hip_atomic_store(&sf->dig[0][0] + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          row_barrier(hdr, G, nbar, p.sync);
        }
      }
    }
    if (path == 1 || path == 5) {
      // ---- compaction (a6) --------------------------------------------------
      // Waves 0 and 1 find the edges of b* and b* + 1; wave 2 sums, over the
      // workgroups before this one, their winners (scores in bins > b*) and
      // members (scores in b*) from their slices: this workgroup's winners
      // take output slots from the first sum on, its members list slots
      // from the second.
      if (w < 2) {
        const float e = bin_edge(cr.b + w, bm);
        if (l == 0) sm.thr[w] = w == 0 ? fmaxf(e, xfloor) : e;
      } else if (w == 2) {
        uint32_t s0 = 0u, s1 = 0u;
        if (l < g) {
          const uint16_t* sl = slices + (size_t)l * kBins;
          if (cr.b + 1 < kBins)
            s1 = __hip_atomic_load(&sl[cr.b + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          s0 = __hip_atomic_load(&sl[cr.b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint32_t ow = wave_incl_scan(s1);
        const uint32_t om = wave_incl_scan(s0 - s1);
        if (l == 63) {
          sm.bc[0] = ow;
          sm.bc[1] = om;
        }
      }
      lds_sync();
      const uint32_t need = (uint32_t)K - cr.above;
      const uint32_t m = cr.m;
      const uint32_t above = cr.above;
      const bool direct = need == m;  // every member is selected
      uint32_t wb[NW], cb[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) wb[i] = cb[i] = 0u;
      // this thread's winner (x >= x_hi) and member (x_lo <= x < x_hi) bits,
      // shifted in group by group
      int ngrp = 0;  // groups this wave visited (uniform)
      {
        const float xlo = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.thr[0])));
        const float xhi = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.thr[1])));
        each([&](int j, int q, bool) {
          group_bits(v[j], xlo, xhi, wb[j >> 3], cb[j >> 3]);
          ngrp = j + 1;
        });
      }
      // word d holds groups 8d .. 8d + 7, nd bits shifted in: bit p is this
      // thread's score i = 32 d + nd - 1 - p (group i / 4, lane i % 4)
      auto nbits = [&](int d) { return 4 * min(max(ngrp - 8 * d, 0), 8); };
      uint32_t nwin = 0, ncand = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        nwin += __popc(wb[i]);
        ncand += __popc(cb[i]);
      }
      const uint32_t ex = wave_offsets((ncand << 16) | nwin, &sm.ctr[2]);
      uint64_t* list = reinterpret_cast<uint64_t*>(s_pair);
      if (__any(ncand != 0u)) {
        uint32_t cpos = sm.bc[1] + (ex >> 16);
        each([&](int j, int q, bool) {
          const int d = j >> 3;
          const int sh = nbits(d) - 4 - 4 * (j - 8 * d);  // the group's lowest bit (score 3)
          const uint32_t cq = (cb[d] >> sh) & 0xFu;
          if (__any(cq != 0u)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool c = (cq >> (3 - e)) & 1u;
              if (c && cpos < m) {
                const int32_t idx = (q << 2) + e - lead;
                if (direct) {
                  store_nt(out + above + cpos, idx);
                } else {
                  float x = v[j][e];
                  asm volatile("" : "+v"(x));
                  const uint64_t pr = ((uint64_t)(uint32_t)idx << 32) | fkey(x);
                  __hip_atomic_store(&list[cpos], pr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
              }
              cpos += c ? 1u : 0u;
            }
          }
        });
      }
      // ---- refine (a7): the row's last part picks `need` members ----------
      // Every workgroup counts itself done once its member-list entries have
      // completed (an add without return: a returning one's round trip is
      // the longer), then writes its winners (nothing reads them in this
      // launch, so their stores overlap the count's round trip).  The row's
      // last part waits for the count to reach G -- a bounded wait, like
      // the row barrier's -- and refines.
      wait_vm();
      __syncthreads();
      if (t == 0) atomic_add_agent_nr(&hdr->done, 1u);
      const bool last = g == G - 1;
      {
        uint32_t wpos = sm.bc[0] + (ex & 0xFFFFu);
        const int base = ((q0 + t) << 2) - lead;
#pragma unroll
        for (int d = 0; d < NW; ++d) {
          const int nb = nbits(d);  // uniform
          if (nb == 0) break;
          uint32_t bits = wb[d] << (32 - nb);
          const int bd = base + 32 * d * BLOCK;
          while (bits) {
            const uint32_t c = walk_pop(bits);
            // (the slot is clamped, not tested: the row's winners number
            // exactly `above` <= K)
            store_nt(out + min(wpos, (uint32_t)K - 1u), bd + walk_offset<BLOCK>(c));
            ++wpos;
          }
        }
      }
      if (!last) return;
      if (t == 0) {
        uint32_t spins = 0;
        while (load_agent(&hdr->done) < (uint32_t)G) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > p.sync.spins) {
            atomic_add_agent_nr(p.sync.err, 1u);
            break;
          }
        }
      }
      __syncthreads();
      if (!direct) {
        for (uint32_t i0 = 0; i0 < m; i0 += 4 * BLOCK) {
          uint64_t r[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t i = i0 + t + u * BLOCK;
            r[u] = i < m ? __hip_atomic_load(&list[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0ull;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t i = i0 + t + u * BLOCK;
            if (i < m) {
              sm.u.c.key[i] = (uint32_t)r[u];
              sm.u.c.idx[i] = (int32_t)(r[u] >> 32);
            }
          }
        }
        lds_sync();
        if (m <= (uint32_t)kRankMax) {
          rank_select_direct<BLOCK>(sm.u.c.key, sm.u.c.idx, m, need, out, above);
        } else {
          list_select<BLOCK>(sm.u.c.key, sm.u.c.idx, m, need, p.deterministic != 0, out, above,
                             (uint32_t)K, sm.dh, &sm.cross, sm.scan, sm.mm, sm.ctr, nbar);
        }
      }
      // back to zero: the histogram bins the first round added to, and the
      // digit rows when a second round used them
      rest_slot(sf, t, BLOCK, blo, path == 5);
      put_stats(path, (int)cr.m, (int)cr.above, cr.b);
      return;
    }
  }

  // ---- rescue (a8): exact radix select over the whole row -----------------
  {
    const RSel s = radix_select<BLOCK, true, SPLIT>(
        resident, (uint32_t)K, sm.dh, &sm.cross, sm.scan, sm.mm,
        SPLIT ? &sf->dig[0][0] : nullptr, SPLIT ? &hdr->class_ext[0] : nullptr, hdr, G, nbar,
        p.sync);
    // Deterministic mode: when the K-th key's class holds more scores than
    // are needed, keep its smallest positions -- a second radix select over
    // the class's complemented positions (other scores count as key 0; the
    // row's workgroups merge through digit rows 4..7).  Positions are
    // distinct, so that select always ends with its last digit class needed
    // whole: the choice takes no ticket.
    const bool pick = p.deterministic && s.cnt > s.rem;
    RSel s2{0u, 0, 0u, 0u};
    if (pick) {
      const uint32_t tkey = s.thr;  // the select ended on one exact key
      s2 = radix_select<BLOCK, true, SPLIT>(
          [&](auto&& f) {
            each([&](int j, int q, bool) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float x = v[j][e];
                asm volatile("" : "+v"(x));
                const uint32_t pos = (uint32_t)((q << 2) + e - lead);
                f(rkey(x) == tkey ? ~pos : 0u);
              }
            });
          },
          s.rem, sm.dh, &sm.cross, sm.scan, sm.mm, SPLIT ? &sf->dig[4][0] : nullptr,
          SPLIT ? &hdr->class_ext[8] : nullptr, hdr, G, nbar, p.sync);
    }
    // a score of the K-th key's class is taken when the tie pick keeps it
    auto kept = [&](int32_t idx) {
      return !pick || (((~(uint32_t)idx) >> s2.shift) >= s2.thr);
    };
    uint32_t ngt = 0, neq = 0;
    each([&](int j, int q, bool) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t d = rkey(v[j][e]) >> s.shift;
        ngt += (d > s.thr) ? 1u : 0u;
        neq += (d == s.thr && kept((q << 2) + e - lead)) ? 1u : 0u;
      }
    });
    if (t == 0) sm.bc[3] = s.thr;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<BLOCK>((neq << 16) | ngt, sm.scan, tot);
    uint32_t gbase = 0, ebase = 0;
    if (SPLIT) {
      if (t == 0) {
        sm.bc[0] = atomic_add_agent(&hdr->win_cur, tot & 0xFFFFu);
        sm.bc[1] = atomic_add_agent(&hdr->tie_cur, tot >> 16);
      }
      lds_sync();
      gbase = sm.bc[0];
      ebase = sm.bc[1];
    }
    uint32_t gpos = gbase + (ex & 0xFFFFu);
    uint32_t tk = ebase + (ex >> 16);
    const uint32_t eqbase = (uint32_t)K - s.rem;
    // re-read after the scan's barriers so the counting pass's compares are
    // not kept live across it
    const uint32_t thr2 = sm.bc[3];
    each([&](int j, int q, bool) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t d = rkey(v[j][e]) >> s.shift;
        const int32_t idx = (q << 2) + e - lead;
        const bool gt = d > thr2;
        const bool eq = d == thr2 && kept(idx);
        if (gt && gpos < (uint32_t)K) store_nt(out + gpos, idx);
        if (eq && tk < s.rem) store_nt(out + eqbase + tk, idx);
        gpos += gt ? 1u : 0u;
        tk += eq ? 1u : 0u;
      }
    });
    bool last = true;
    if (SPLIT) {
      last = finish_slot(hdr, G, &sm.bc[2]);
      if (last) rest_slot(sf, t, BLOCK, 0, true);
    }
    if (last)
      put_stats(path, bracket_ok && !SPLIT ? (int)cr.m : -1, bracket_ok && !SPLIT ? (int)cr.above : -1,
                bracket_ok && !SPLIT ? cr.b : -1);
  }
}

template <int K, int QPT, int BLOCK, bool SPLIT>
__global__ void __launch_bounds__(BLOCK)
    __attribute__((amdgpu_waves_per_eu(WavesPerEu<K, QPT, BLOCK, SPLIT>::value)))
    gvr_topk_kernel(const GvrParams p) {
  __shared__ Smem<K, BLOCK> sm;
  const int G = SPLIT ? p.wgs_per_row : 1;

  // ---- workgroup -> (row slot, part) ------------------------------------
  int slot, g;
  if (SPLIT) {
    int L = blockIdx.x;
    if (p.xcd_group) {
      // Workgroups are dispatched round-robin over the 8 XCDs; renumber so a
      // row's G workgroups are consecutive within one XCD's sequence.
      const int per = gridDim.x >> 3;
      L = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    }
    slot = L / G;
    g = L - slot * G;
  } else {
    // Last row first: in a causal prefill tile a request's windows grow row
    // by row, so its long rows start early and the launch drains on short
    // ones (longest-first dispatch; decode batches of random lengths are
    // indifferent to the order).  Measured on the 4096 x 16640 tile:
    // 40.2 -> 38.2 us.
    slot = (int)gridDim.x - 1 - (int)blockIdx.x;
    g = 0;
  }
  if (slot >= p.rows) return;
  RowCtx c;
  f4 v[QPT];
  float smp[spw<K, BLOCK>()];
  if (!row_begin<K, QPT, BLOCK, SPLIT>(p, sm, slot, g, c, v, smp)) return;
  row_finish<K, QPT, BLOCK, SPLIT>(p, sm, g, c, v, smp);
}

// ---------------------------------------------------------------------------
// Host-side dispatch over the instantiated shapes
// ---------------------------------------------------------------------------

template <int K, int QPT, int BLOCK, bool SPLIT>
static const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&gvr_topk_kernel<K, QPT, BLOCK, SPLIT>);
}

template <int K>
static const void* pick(int block, int qpt, bool split) {
  if (split) {
    if (block == 256 && qpt == 4) return kernel_ptr<K, 4, 256, true>();
    if (block == 256 && qpt == 8) return kernel_ptr<K, 8, 256, true>();
    if (block == 512 && qpt == 9) return kernel_ptr<K, 9, 512, true>();
    return nullptr;
  }
  if (block == 256 && qpt == 8) return kernel_ptr<K, 8, 256, false>();
  if (block == 256 && qpt == 17) return kernel_ptr<K, 17, 256, false>();
  if (block == 512 && qpt == 9) return kernel_ptr<K, 9, 512, false>();
  if (block == 1024 && qpt == 9) return kernel_ptr<K, 9, 1024, false>();
  return nullptr;
}

const void* gvr_kernel(int k, int block, int qpt, bool split) {
  switch (k) {
    case 512: return pick<512>(block, qpt, split);
    case 1024: return pick<1024>(block, qpt, split);
    case 2048: return pick<2048>(block, qpt, split);
    default: return nullptr;
  }
}

}  // namespace ert
