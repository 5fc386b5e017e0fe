// gvr_kernels.hip -- gfx950 kernels of the exact per-row top-K
// (Guess-Verify-Refine with block64 sampling and an exact radix rescue).
//
// One fused kernel template serves both tiers:
//  * one workgroup per row (SPLIT = false): the row is resident in the
//    workgroup's VGPRs, every merge happens in LDS, nothing is shared across
//    workgroups;
//  * G workgroups per row (SPLIT = true): each workgroup keeps 1/G of the row
//    resident in VGPRs; histograms merge through a per-row workspace slot with
//    agent-scope atomics and a generation barrier, candidates are appended to
//    the slot, and the last workgroup to finish refines them and cleans the
//    slot so the next call (or graph replay) finds it zeroed.
//
// Steps per long row (nv > K), following PR 20998 "Why the GLM row overflows"
// and "What changes" (TensorRT-LLM, "GVR K=2048 reg_clus with block64 sampling
// and parallel rescue"):
//  1. load the row once, as aligned float4 groups starting at col0 = ks & ~3,
//     with lanes outside [ks, ke) masked by position (PR 18702 "Kernel": never
//     a materialised -inf);
//  2. guess: K/64 blocks of 64 consecutive scores spread over the valid window
//     including both ends; the bracket is their min / max;
//  3. verify: histogram the row over kBins bins of the bracket (scores beyond
//     the bracket clamp into the end bins); an invalid bracket (non-finite or
//     collapsed) skips to the rescue;
//  4. the crossing bin b*: the highest bin whose count from the top reaches K;
//     everything above it is selected, b* holds m candidates of which
//     need = K - above are selected;
//  5. compact winners straight to the output and candidates to a buffer;
//  6. refine: exact radix select of the `need` largest candidate keys;
//  7. rescue when the bracket is invalid or m exceeds the candidate cap: an
//     exact 4 x 8-bit radix select over the whole row's resident keys, using
//     every workgroup of the row, inside the same launch.
//
// Ordering: scores compare as IEEE values with -0 == +0; the order-preserving
// key maps a float to a uint32 whose unsigned order is that value order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gvr_common.h"

namespace ert {

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------

// Order-preserving key: canonicalise -0 to +0, then flip so unsigned order
// matches IEEE order (negatives inverted, positives get the top bit).
__device__ __forceinline__ uint32_t fkey(float x) {
  uint32_t b = __float_as_uint(x);
  b = (b == 0x80000000u) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Histogram bin of x over the bracket: clamp((x - gmin) * sc, 0, kBins - 1),
// truncated.  Monotone non-decreasing in x, equal values share a bin, and it
// is the single definition every pass uses (the build disables FP
// contraction, so no pass can compute it differently).  The final mask only
// matters for NaN (outside the contract): it keeps the LDS index in range.
__device__ __forceinline__ int vbin(float x, float gmin, float sc) {
  float t = (x - gmin) * sc;
  t = __builtin_amdgcn_fmed3f(t, 0.0f, (float)(kBins - 1));
  return ((int)t) & (kBins - 1);
}

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float comp(const f4& v, int e) { return v[e]; }

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Block primitives (kBlock threads = kWaves wave64s)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t n = __shfl_up(v, d, 64);
    if (l >= d) v += n;
  }
  return v;
}

// Exclusive prefix sum over the block in thread order; `total` gets the sum.
// `sm` holds kWaves words.  Contains two __syncthreads.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sm, uint32_t& total) {
  const uint32_t inc = wave_incl_scan(v);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 63) sm[w] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t s = sm[i];
    off += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

struct Cross {
  int b;           // crossing bin / digit, -1 if the total is below target
  uint32_t above;  // count strictly above it
  uint32_t m;      // count inside it
  uint32_t total;
};

// Find the highest bin b with sum_{b' >= b} h[b'] >= target over NBINS bins,
// where load(b) returns h[b].  Thread t owns NBINS/kBlock consecutive bins
// from the top.  Result in *out (LDS), visible to all threads on return.
template <int NBINS, class Load>
__device__ __forceinline__ void find_crossing(Load load, uint32_t target, Cross* out, uint32_t* scan_sm) {
  constexpr int PER = NBINS / kBlock;
  static_assert(PER * kBlock == NBINS, "bins per thread");
  const int t = threadIdx.x;
  const int hi = NBINS - 1 - t * PER;
  uint32_t c[PER];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = load(hi - i);
    s += c[i];
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan(s, scan_sm, tot);
  if (ex < target && ex + s >= target) {
    uint32_t run = ex;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (run + c[i] >= target) {
        out->b = hi - i;
        out->above = run;
        out->m = c[i];
        out->total = tot;
        break;
      }
      run += c[i];
    }
  }
  if (t == 0 && tot < target) {
    out->b = -1;
    out->above = tot;
    out->m = 0;
    out->total = tot;
  }
  __syncthreads();
}

// Generation barrier over the G workgroups of one row (split tier).  The
// generation is read (acquire) before arriving, so a workgroup can never read
// the flipped value of its own barrier instance.  Spins are bounded: on
// timeout an error flag is raised in the workspace and the workgroup moves on
// (results are then undefined, but every wave exits).
__device__ __forceinline__ void row_barrier(SlotHeader* hdr, int G, uint32_t* err) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t gen = __hip_atomic_load(&hdr->bar_gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t arrived = atomic_add_agent(&hdr->bar_count, 1u);
    if (arrived == (uint32_t)(G - 1)) {
      __hip_atomic_store(&hdr->bar_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&hdr->bar_gen, gen + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      uint32_t spins = 0;
      while (load_agent(&hdr->bar_gen) == gen) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > (1u << 24)) {
          atomic_add_agent(err, kErrBarrierTimeout);
          break;
        }
      }
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <int K, int QPT, bool SPLIT>
struct Smem {
  static constexpr int kCap = SPLIT ? 1 : kSingleCap;
  union {
    uint32_t hist[kBins];
    struct {
      uint32_t key[kCap];
      int32_t idx[kCap];
    } c;
  } u;
  uint32_t dh[256];
  uint32_t scan[kWaves];
  float rmin[kWaves];
  float rmax[kWaves];
  Cross cross;
  uint32_t ctr[4];
  uint32_t bc[4];
};

template <int K, int QPT, bool SPLIT>
__global__ void __launch_bounds__(kBlock) gvr_topk_kernel(const GvrParams p) {
  constexpr int NSB = K / 64;   // sample blocks
  constexpr int NEL = QPT * 4;  // resident elements per thread
  constexpr int NW = (NEL + 31) / 32;
  __shared__ Smem<K, QPT, SPLIT> sm;

  const int t = threadIdx.x;
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
    slot = blockIdx.x;
    g = 0;
  }
  if (slot >= p.rows) return;
  const int64_t row = (int64_t)p.row_begin + slot;

  // ---- row resolve (a0) ---------------------------------------------------
  const int64_t S = p.row_stride;
  int64_t ks, nv;
  if (p.n_valid) {
    int64_t n = p.n_valid[row];
    ks = 0;
    nv = n < 0 ? 0 : (n > S ? S : n);
  } else {
    int64_t a = p.row_starts[row], e = p.row_ends[row];
    a = a < 0 ? 0 : (a > S ? S : a);
    e = e < a ? a : (e > S ? S : e);
    ks = a;
    nv = e - a;
  }
  int32_t* out = p.indices + row * K;
  int32_t* stats = p.row_stats ? p.row_stats + row * kStatsWords : nullptr;

  // ---- short row (a1): identity then -1 ----------------------------------
  if (nv <= K) {
    for (int i = g * kBlock + t; i < K; i += G * kBlock) out[i] = (i < nv) ? i : -1;
    if (stats && g == 0 && t < kStatsWords)
      stats[t] = (t == 0) ? 0 : (t == 6 ? G : (t == 7 ? p.cap : -1));
    return;
  }

  // ---- part of the row this workgroup owns -------------------------------
  const int64_t col0 = ks & ~(int64_t)3;
  const int lead = (int)(ks & 3);
  const int64_t span = lead + nv;     // positions [0, span) from col0
  const int64_t Q = (span + 3) >> 2;  // float4 groups
  int64_t q0 = 0, q1 = Q;
  if (SPLIT) {
    const int64_t Qp = (Q + G - 1) / G;
    q0 = (int64_t)g * Qp;
    q1 = q0 + Qp < Q ? q0 + Qp : Q;
  }
  const float* rowp = p.logits + row * S;
  const f4* base = reinterpret_cast<const f4*>(rowp + col0);

  unsigned char* sb = nullptr;
  SlotHeader* hdr = nullptr;
  uint32_t* s_hist = nullptr;
  uint32_t* s_dig = nullptr;
  uint32_t* s_key = nullptr;
  int32_t* s_idx = nullptr;
  uint32_t* err = nullptr;
  if (SPLIT) {
    sb = p.ws + kWsHeaderBytes + (size_t)slot * kSlotBytes;
    hdr = reinterpret_cast<SlotHeader*>(sb);
    s_hist = reinterpret_cast<uint32_t*>(sb + kSlotHistOff);
    s_dig = reinterpret_cast<uint32_t*>(sb + kSlotDigitOff);
    s_key = reinterpret_cast<uint32_t*>(sb + kSlotKeyOff);
    s_idx = reinterpret_cast<int32_t*>(sb + kSlotIdxOff);
    err = reinterpret_cast<uint32_t*>(p.ws);
  }

  const int w = t >> 6;
  const int l = lane_id();

  // ---- guess (a3): block64 sample over the valid window -------------------
  // Block j starts at floor(j * (nv - 64) / (NSB - 1)); blocks are disjoint
  // for nv > K, so the sample holds exactly K distinct scores, and the first
  // and last blocks touch both ends of the window.
  float smin = __builtin_inff(), smax = -__builtin_inff();
  {
    const float* win = rowp + ks;
#pragma unroll
    for (int j = w; j < NSB; j += kWaves) {
      const int64_t st = ((int64_t)j * (nv - 64)) / (NSB - 1);
      const float x = win[st + l];
      smin = fminf(smin, x);
      smax = fmaxf(smax, x);
    }
  }

  // ---- scan (a2): the part, resident in VGPRs -----------------------------
  f4 v[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int64_t q = q0 + t + (int64_t)j * kBlock;
    if (q < q1) {
      v[j] = __builtin_nontemporal_load(base + q);
    } else {
      v[j] = f4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // Positional validity of the four lanes of resident group j.
  auto qmask = [&](int j) -> uint32_t {
    const int64_t q = q0 + t + (int64_t)j * kBlock;
    if (q >= q1) return 0u;
    const int64_t p0 = q << 2;
    uint32_t m = 0xFu;
    if (p0 < lead) m &= (0xFu << (lead - p0)) & 0xFu;
    const int64_t rem = span - p0;
    if (rem < 4) m &= (1u << rem) - 1u;
    return m;
  };
  // Local-frame index of lane e of group j.
  auto lidx = [&](int j, int e) -> int32_t {
    const int64_t q = q0 + t + (int64_t)j * kBlock;
    return (int32_t)((q << 2) + e - lead);
  };

#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    smin = fminf(smin, __shfl_xor(smin, o, 64));
    smax = fmaxf(smax, __shfl_xor(smax, o, 64));
  }
  if (l == 0) {
    sm.rmin[w] = smin;
    sm.rmax[w] = smax;
  }
  for (int i = t; i < kBins; i += kBlock) sm.u.hist[i] = 0u;
  if (t < 4) sm.ctr[t] = 0u;
  __syncthreads();
  float gmin = sm.rmin[0], gmax = sm.rmax[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) {
    gmin = fminf(gmin, sm.rmin[i]);
    gmax = fmaxf(gmax, sm.rmax[i]);
  }
  const float range = gmax - gmin;
  const float sc = (float)kBins / range;
  const bool bracket_ok = __builtin_isfinite(gmin) && __builtin_isfinite(gmax) && (gmax > gmin) &&
                          __builtin_isfinite(range) && __builtin_isfinite(sc) && (sc > 0.0f) &&
                          !p.force_rescue;

  int path = 2;  // 1 fast, 2 rescue (invalid bracket), 3 rescue (overflow)
  Cross cr{-1, 0u, 0u, 0u};

  // ---- verify (a4, a5): histogram and crossing bin ------------------------
  if (bracket_ok) {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const uint32_t m = qmask(j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((m >> e) & 1u) {
          const int b = vbin(comp(v[j], e), gmin, sc);
          __hip_atomic_fetch_add(&sm.u.hist[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
    __syncthreads();
    if (SPLIT) {
      for (int b = t; b < kBins; b += kBlock) {
        const uint32_t c = sm.u.hist[b];
        if (c) atomic_add_agent(&s_hist[b], c);
      }
      row_barrier(hdr, G, err);
      find_crossing<kBins>([&](int b) { return load_agent(&s_hist[b]); }, (uint32_t)K, &sm.cross,
                           sm.scan);
    } else {
      find_crossing<kBins>([&](int b) { return sm.u.hist[b]; }, (uint32_t)K, &sm.cross, sm.scan);
    }
    cr = sm.cross;
    path = (cr.b >= 0 && cr.m <= (uint32_t)p.cap) ? 1 : 3;
  }

  if (path == 1) {
    // ---- compaction (a6) --------------------------------------------------
    const uint32_t need = (uint32_t)K - cr.above;
    uint32_t wm[NW], cm[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) wm[i] = cm[i] = 0u;
    uint32_t nwin = 0, ncand = 0;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const uint32_t m = qmask(j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = j * 4 + e;
        const int b = vbin(comp(v[j], e), gmin, sc);
        const bool ok = (m >> e) & 1u;
        const uint32_t isw = (ok && b > cr.b) ? 1u : 0u;
        const uint32_t isc = (ok && b == cr.b) ? 1u : 0u;
        wm[i >> 5] |= isw << (i & 31);
        cm[i >> 5] |= isc << (i & 31);
        nwin += isw;
        ncand += isc;
      }
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((ncand << 16) | nwin, sm.scan, tot);
    uint32_t wbase = 0, cbase = 0;
    if (SPLIT) {
      if (t == 0) {
        sm.bc[0] = atomic_add_agent(&hdr->win_cur, tot & 0xFFFFu);
        sm.bc[1] = atomic_add_agent(&hdr->cand_cur, tot >> 16);
      }
      __syncthreads();
      wbase = sm.bc[0];
      cbase = sm.bc[1];
    }
    uint32_t wpos = wbase + (ex & 0xFFFFu);
    uint32_t cpos = cbase + (ex >> 16);
    const uint32_t ccap = SPLIT ? (uint32_t)kSplitCapMax : (uint32_t)kSingleCap;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const uint32_t wq = (wm[(j * 4) >> 5] >> ((j * 4) & 31)) & 0xFu;
      const uint32_t cq = (cm[(j * 4) >> 5] >> ((j * 4) & 31)) & 0xFu;
      if (wq | cq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((wq >> e) & 1u) {
            if (wpos < (uint32_t)K) out[wpos] = lidx(j, e);
            ++wpos;
          }
          if ((cq >> e) & 1u) {
            if (cpos < ccap) {
              if (SPLIT) {
                s_key[cpos] = fkey(comp(v[j], e));
                s_idx[cpos] = lidx(j, e);
              } else {
                sm.u.c.key[cpos] = fkey(comp(v[j], e));
                sm.u.c.idx[cpos] = lidx(j, e);
              }
            }
            ++cpos;
          }
        }
      }
    }

    // ---- refine (a7) ------------------------------------------------------
    bool refine_here = !SPLIT;
    if (SPLIT) {
      __syncthreads();
      if (t == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        sm.bc[2] = atomic_add_agent(&hdr->done, 1u);
      }
      __syncthreads();
      refine_here = (sm.bc[2] == (uint32_t)(G - 1));
      if (refine_here) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    } else {
      __syncthreads();
    }
    if (refine_here) {
      const uint32_t m = cr.m;
      const uint32_t* keys = SPLIT ? s_key : sm.u.c.key;
      const int32_t* idxs = SPLIT ? s_idx : sm.u.c.idx;
      // candidates owned by this thread: i = t + k * kBlock, k < CPT
      constexpr int CPT = (SPLIT ? kSplitCapMax : kSingleCap) / kBlock;
      if (need == m) {
        for (uint32_t i = t; i < m; i += kBlock) out[cr.above + i] = idxs[i];
      } else {
        // exact radix select of the `need` largest keys among m candidates
        uint32_t prefix = 0, rem = need;
        int shift = 24;
        for (int L = 0; L < 4; ++L) {
          shift = 24 - 8 * L;
          sm.dh[t] = 0u;
          __syncthreads();
          for (uint32_t i = t; i < m; i += kBlock) {
            const uint32_t key = keys[i];
            if (L == 0 || ((key ^ prefix) >> (shift + 8)) == 0u)
              __hip_atomic_fetch_add(&sm.dh[(key >> shift) & 255u], 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          __syncthreads();
          find_crossing<256>([&](int d) { return sm.dh[d]; }, rem, &sm.cross, sm.scan);
          const Cross c = sm.cross;
          prefix |= (uint32_t)c.b << shift;
          rem -= c.above;
          if (c.m == rem) break;
        }
        // emit: above the threshold digit -> taken; equal -> first `rem` by ticket
        const uint32_t thr = prefix >> shift;
        uint64_t gtm = 0, eqm = 0;
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int k2 = 0; k2 < CPT; ++k2) {
          const uint32_t i = t + (uint32_t)k2 * kBlock;
          if (i < m) {
            const uint32_t d = keys[i] >> shift;
            const uint64_t bit = 1ull << k2;
            if (d > thr) {
              gtm |= bit;
              ++ngt;
            } else if (d == thr) {
              eqm |= bit;
              ++neq;
            }
          }
        }
        uint32_t tot2;
        const uint32_t ex2 = block_excl_scan((neq << 16) | ngt, sm.scan, tot2);
        uint32_t gpos = cr.above + (ex2 & 0xFFFFu);
        uint32_t tk = ex2 >> 16;
        const uint32_t eqbase = cr.above + (need - rem);
#pragma unroll
        for (int k2 = 0; k2 < CPT; ++k2) {
          const uint64_t bit = 1ull << k2;
          const uint32_t i = t + (uint32_t)k2 * kBlock;
          if (gtm & bit) {
            if (gpos < (uint32_t)K) out[gpos] = idxs[i];
            ++gpos;
          } else if (eqm & bit) {
            if (tk < rem) out[eqbase + tk] = idxs[i];
            ++tk;
          }
        }
      }
    }
    if (SPLIT && refine_here) {
      // last workgroup: clean the slot for the next call
      __syncthreads();
      for (int i = t; i < kBins; i += kBlock) s_hist[i] = 0u;
      if (t == 0) {
        hdr->win_cur = 0u;
        hdr->cand_cur = 0u;
        hdr->tie_cur = 0u;
        hdr->done = 0u;
      }
    }
    if (stats && (SPLIT ? refine_here : true) && t == 0) {
      stats[0] = 1;
      stats[1] = (int)cr.m;
      stats[2] = (int)cr.above;
      stats[3] = cr.b;
      stats[4] = (int)__float_as_uint(gmin);
      stats[5] = (int)__float_as_uint(gmax);
      stats[6] = G;
      stats[7] = p.cap;
    }
    return;
  }

  // ---- rescue (a8): exact radix select over the whole row -----------------
  {
    uint32_t prefix = 0, rem = (uint32_t)K;
    int shift = 24;
    for (int L = 0; L < 4; ++L) {
      shift = 24 - 8 * L;
      sm.dh[t] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < QPT; ++j) {
        const uint32_t m = qmask(j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((m >> e) & 1u) {
            const uint32_t key = fkey(comp(v[j], e));
            if (L == 0 || ((key ^ prefix) >> (shift + 8)) == 0u)
              __hip_atomic_fetch_add(&sm.dh[(key >> shift) & 255u], 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
      }
      __syncthreads();
      if (SPLIT) {
        uint32_t* gd = s_dig + L * 256;
        const uint32_t c = sm.dh[t];
        if (c) atomic_add_agent(&gd[t], c);
        row_barrier(hdr, G, err);
        find_crossing<256>([&](int d) { return load_agent(&gd[d]); }, rem, &sm.cross, sm.scan);
      } else {
        find_crossing<256>([&](int d) { return sm.dh[d]; }, rem, &sm.cross, sm.scan);
      }
      const Cross c = sm.cross;
      prefix |= (uint32_t)c.b << shift;
      rem -= c.above;
      if (c.m == rem) break;
    }
    const uint32_t thr = prefix >> shift;
    uint32_t gm[NW], em[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) gm[i] = em[i] = 0u;
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const uint32_t m = qmask(j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = j * 4 + e;
        const uint32_t d = fkey(comp(v[j], e)) >> shift;
        const bool ok = (m >> e) & 1u;
        const uint32_t isg = (ok && d > thr) ? 1u : 0u;
        const uint32_t ise = (ok && d == thr) ? 1u : 0u;
        gm[i >> 5] |= isg << (i & 31);
        em[i >> 5] |= ise << (i & 31);
        ngt += isg;
        neq += ise;
      }
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((neq << 16) | ngt, sm.scan, tot);
    uint32_t gbase = 0, ebase = 0;
    if (SPLIT) {
      if (t == 0) {
        sm.bc[0] = atomic_add_agent(&hdr->win_cur, tot & 0xFFFFu);
        sm.bc[1] = atomic_add_agent(&hdr->tie_cur, tot >> 16);
      }
      __syncthreads();
      gbase = sm.bc[0];
      ebase = sm.bc[1];
    }
    uint32_t gpos = gbase + (ex & 0xFFFFu);
    uint32_t tk = ebase + (ex >> 16);
    const uint32_t eqbase = (uint32_t)K - rem;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const uint32_t gq = (gm[(j * 4) >> 5] >> ((j * 4) & 31)) & 0xFu;
      const uint32_t eq = (em[(j * 4) >> 5] >> ((j * 4) & 31)) & 0xFu;
      if (gq | eq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((gq >> e) & 1u) {
            if (gpos < (uint32_t)K) out[gpos] = lidx(j, e);
            ++gpos;
          }
          if ((eq >> e) & 1u) {
            if (tk < rem) out[eqbase + tk] = lidx(j, e);
            ++tk;
          }
        }
      }
    }
    bool last = true;
    if (SPLIT) {
      __syncthreads();
      if (t == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        sm.bc[2] = atomic_add_agent(&hdr->done, 1u);
      }
      __syncthreads();
      last = (sm.bc[2] == (uint32_t)(G - 1));
      if (last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        for (int i = t; i < kBins; i += kBlock) s_hist[i] = 0u;
        for (int i = t; i < 4 * 256; i += kBlock) s_dig[i] = 0u;
        if (t == 0) {
          hdr->win_cur = 0u;
          hdr->cand_cur = 0u;
          hdr->tie_cur = 0u;
          hdr->done = 0u;
        }
      }
    }
    if (stats && last && t == 0) {
      stats[0] = path;
      stats[1] = bracket_ok ? (int)cr.m : -1;
      stats[2] = bracket_ok ? (int)cr.above : -1;
      stats[3] = bracket_ok ? cr.b : -1;
      stats[4] = (int)__float_as_uint(gmin);
      stats[5] = (int)__float_as_uint(gmax);
      stats[6] = G;
      stats[7] = p.cap;
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch over the instantiated shapes
// ---------------------------------------------------------------------------

template <int K, int QPT, bool SPLIT>
static const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&gvr_topk_kernel<K, QPT, SPLIT>);
}

template <int K, bool SPLIT>
static const void* pick_qpt(int qpt) {
  switch (qpt) {
    case 4: return kernel_ptr<K, 4, SPLIT>();
    case 8: return kernel_ptr<K, 8, SPLIT>();
    case 17: return kernel_ptr<K, 17, SPLIT>();
    default: return nullptr;
  }
}

const void* gvr_kernel(int k, int qpt, bool split) {
  switch (k) {
    case 512: return split ? pick_qpt<512, true>(qpt) : pick_qpt<512, false>(qpt);
    case 1024: return split ? pick_qpt<1024, true>(qpt) : pick_qpt<1024, false>(qpt);
    case 2048: return split ? pick_qpt<2048, true>(qpt) : pick_qpt<2048, false>(qpt);
    default: return nullptr;
  }
}

}  // namespace ert
