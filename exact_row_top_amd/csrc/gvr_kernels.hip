// gvr_kernels.hip -- gfx950 kernels of the exact per-row top-K
// (Guess-Verify-Refine with block64 sampling and an exact radix rescue).
//
// One fused kernel template serves both tiers:
//  * one workgroup per row (SPLIT = false): the row is resident in the
//    workgroup's VGPRs, every merge happens in LDS, nothing is shared across
//    workgroups;
//  * G workgroups per row (SPLIT = true): each workgroup keeps 1/G of the row
//    resident in VGPRs.  Histograms merge through a per-row workspace slot
//    (dense per-workgroup slices, summed by every workgroup after a
//    generation barrier), candidates are appended to the slot, and the last
//    workgroup to finish refines them and clears the slot's counters so the
//    next call (or graph replay) finds them at rest.
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
//  5. compact winners straight to the output and candidates to a buffer;
//  6. refine: the `need` largest candidates, exactly;
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

typedef float f4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float from_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Rescue key: fkey, with every NaN (the masked-lane marker) mapped to 0, the
// lowest key, so it sits below -inf (key 0x007FFFFF) and is never selected
// while the row holds K non-NaN scores.
__device__ __forceinline__ uint32_t rkey(float x) { return (x == x) ? fkey(x) : 0u; }

// Histogram bin of x over the bracket: clamp((x - gmin) * sc, 0, kBins - 1),
// truncated.  Monotone non-decreasing in x, equal values share a bin, and it
// is the single definition every step uses (the build disables FP
// contraction, so no step can evaluate it differently).  The final mask only
// matters for NaN (outside the contract): it keeps the LDS index in range.
__device__ __forceinline__ int vbin(float x, float gmin, float sc) {
  float t = (x - gmin) * sc;
  t = __builtin_amdgcn_fmed3f(t, 0.0f, (float)(kBins - 1));
  return ((int)t) & (kBins - 1);
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void lds_inc(uint32_t* p) {
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------------------
// Wave and block primitives (kBlock threads = kWaves wave64s)
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts
// (within rows of 16) and the gfx9 row broadcasts (across rows).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int l = lane_id();
  const int rl = l & 15;
  uint32_t s;
  s = dpp_u32<0x111>(v);
  v += (rl >= 1) ? s : 0u;
  s = dpp_u32<0x112>(v);
  v += (rl >= 2) ? s : 0u;
  s = dpp_u32<0x114>(v);
  v += (rl >= 4) ? s : 0u;
  s = dpp_u32<0x118>(v);
  v += (rl >= 8) ? s : 0u;
  s = dpp_u32<0x142>(v);
  v += ((l & 31) >= 16) ? s : 0u;
  s = dpp_u32<0x143>(v);
  v += (l >= 32) ? s : 0u;
  return v;
}

// Min and max over a wave (result in every lane, read from lane 63).
__device__ __forceinline__ void wave_minmax(float& mn, float& mx) {
  const int l = lane_id();
  const int rl = l & 15;
  float a, b;
#define ERT_STEP(CTRL, COND) \
  a = dpp_f32<CTRL>(mn);     \
  b = dpp_f32<CTRL>(mx);     \
  if (COND) {                \
    mn = fminf(mn, a);       \
    mx = fmaxf(mx, b);       \
  }
  ERT_STEP(0x111, rl >= 1)
  ERT_STEP(0x112, rl >= 2)
  ERT_STEP(0x114, rl >= 4)
  ERT_STEP(0x118, rl >= 8)
  ERT_STEP(0x142, (l & 31) >= 16)
  ERT_STEP(0x143, l >= 32)
#undef ERT_STEP
  mn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mn), 63));
  mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 63));
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
__device__ __forceinline__ void find_crossing(Load load, uint32_t target, Cross* out,
                                              uint32_t* scan_sm) {
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
    bool found = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!found && run + c[i] >= target) {
        out->b = hi - i;
        out->above = run;
        out->m = c[i];
        out->total = tot;
        found = true;
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

// Smallest score x (IEEE order over [-inf, +inf]) with vbin(x) >= b, so that
// for every non-NaN x: vbin(x) >= b  <=>  x >= edge.  vbin is monotone in x,
// so the set is an up-set; a 64-way search over the order-preserving keys of
// -inf .. +inf (each round probes 64 evenly spaced keys, one per lane) finds
// its least element in six rounds.  b <= 0 gives -inf; b >= kBins gives NaN,
// which no score compares >= to.  Must be called by a whole wave.
__device__ __forceinline__ float bin_edge(int b, float gmin, float sc) {
  if (b <= 0) return -__builtin_inff();
  if (b >= kBins) return __builtin_nanf("");
  uint32_t lo = 0x007FFFFFu;  // key(-inf): vbin = 0 < b
  uint32_t hi = 0xFF800000u;  // key(+inf): vbin = kBins - 1 >= b
  const uint32_t l = (uint32_t)lane_id();
  while (hi - lo > 1u) {
    const uint32_t span = hi - lo;
    const uint32_t step = span / 64u + ((span & 63u) ? 1u : 0u);
    const uint64_t pk = (uint64_t)lo + (uint64_t)(l + 1u) * step;
    const uint32_t probe = pk >= (uint64_t)hi ? hi : (uint32_t)pk;
    const bool ok = vbin(from_key(probe), gmin, sc) >= b;
    const uint64_t mask = __ballot(ok);  // lane 63 probes hi, so mask != 0
    const int f = __ffsll((unsigned long long)mask) - 1;
    const uint32_t nhi = __shfl(probe, f, 64);
    const uint32_t nlo = (f > 0) ? __shfl(probe, f - 1, 64) : lo;
    lo = nlo;
    hi = nhi;
  }
  return from_key(hi);
}

// Generation barrier over the G workgroups of one row (split tier).  The
// generation is read (acquire) before arriving, so a workgroup can never read
// the flipped value of its own barrier instance.  Spins are bounded: on
// timeout an error flag is raised in the workspace and the workgroup moves on
// (results are then undefined, but every wave exits).
__device__ __forceinline__ void row_barrier(SlotHeader* hdr, int G, uint32_t* err) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t gen =
        __hip_atomic_load(&hdr->bar_gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t arrived = atomic_add_agent(&hdr->bar_count, 1u);
    if (arrived == (uint32_t)(G - 1)) {
      __hip_atomic_store(&hdr->bar_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&hdr->bar_gen, gen + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      uint32_t spins = 0;
      while (load_agent(&hdr->bar_gen) == gen) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1u << 25)) {
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

constexpr int kRankMax = kBlock;  // refine by rank counting up to this many candidates

template <int K, int QPT, bool SPLIT>
struct Smem {
  static constexpr int kCap = SPLIT ? kRankMax : kSingleCap;
  union {
    uint32_t hist[kBins + 64];  // + one trash word per lane for NaN markers
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
  float thr[2];
  uint32_t bc[4];
};

template <int K, int QPT, bool SPLIT>
__global__ void __launch_bounds__(kBlock) gvr_topk_kernel(const GvrParams p) {
  constexpr int NSB = K / 64;        // sample blocks
  constexpr int SPW = NSB / kWaves;  // sample blocks per wave
  constexpr int NW = (QPT * 4 + 31) / 32;
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

  // ---- row resolve (a0); row_stride < 2^30 is checked on the host --------
  const int S = (int)p.row_stride;
  int ks, nv;
  if (p.n_valid) {
    const int n = p.n_valid[row];
    ks = 0;
    nv = n < 0 ? 0 : (n > S ? S : n);
  } else {
    int a = p.row_starts[row], e = p.row_ends[row];
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

  SlotHeader* hdr = nullptr;
  uint32_t* s_key = nullptr;
  int32_t* s_idx = nullptr;
  uint32_t* s_wh = nullptr;  // [G][kBins]
  uint32_t* s_wd = nullptr;  // [G][4][256]
  uint32_t* err = nullptr;
  if (SPLIT) {
    hdr = reinterpret_cast<SlotHeader*>(p.ws + kWsHeaderBytes) + slot;
    unsigned char* sb = p.ws + kWsDataOff + (size_t)slot * p.slot_data_bytes;
    s_key = reinterpret_cast<uint32_t*>(sb + kSlotKeyOff);
    s_idx = reinterpret_cast<int32_t*>(sb + kSlotIdxOff);
    s_wh = reinterpret_cast<uint32_t*>(sb + kSlotWgHistOff);
    s_wd = s_wh + (size_t)G * kBins;
    err = reinterpret_cast<uint32_t*>(p.ws);
  }

  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, uniform
  const int l = lane_id();

  // ---- guess (a3): block64 sample over the valid window -------------------
  // Block j starts at floor(j * (nv - 64) / (NSB - 1)); blocks are disjoint
  // for nv > K, so the sample holds exactly K distinct scores, and the first
  // and last blocks touch both ends of the window.  Wave w reads blocks
  // w, w + kWaves, ...: one 256-byte load per block.
  float smp[SPW];
  {
    const float* win = rowp + ks;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int j = w + i * kWaves;
      const int st = (int)(((int64_t)j * (nv - 64)) / (NSB - 1));
      smp[i] = win[st + l];
    }
  }

  // ---- scan (a2): the part, resident in VGPRs -----------------------------
  // Thread t holds groups q0 + t + j * kBlock, j < QPT: each load instruction
  // of a wave reads 1 KiB of consecutive scores.  Lanes outside the window or
  // the part (the <= 3 lead lanes, the tail of the last group, groups past the
  // part) become NaN markers here: no selection step accepts a NaN (its
  // compares are false, its histogram increment goes to a trash word, its
  // rescue key is the lowest key), and a genuine -inf tie class stays intact.
  const float qnan = __builtin_nanf("");
  f4 v[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int q = q0 + t + j * kBlock;
    if (q < q1) {
      v[j] = __builtin_nontemporal_load(base + q);
    } else {
      v[j] = f4{qnan, qnan, qnan, qnan};
    }
  }
  {
    // first group of the window (lead lanes): q == 0 is thread 0's j == 0
    if (q0 == 0 && t == 0 && lead > 0) {
#pragma unroll
      for (int e = 0; e < 3; ++e)
        if (e < lead) v[0][e] = qnan;
    }
    // last group of the window (tail lanes), if it lies in this part
    const int qlast = Q - 1;
    const int tail = span - (qlast << 2);  // valid lanes in the last group, 1..4
    if (tail < 4 && qlast >= q0 && qlast < q1) {
      const int d = qlast - q0;
      if ((d % kBlock) == t) {
        const int jl = d / kBlock;
#pragma unroll
        for (int j = 0; j < QPT; ++j)
          if (j == jl) {
#pragma unroll
            for (int e = 1; e < 4; ++e)
              if (e >= tail) v[j][e] = qnan;
          }
      }
    }
  }
  // Visit this thread's groups; `full` (uniform per wave) says all 64 lanes
  // hold four in-window scores, so only boundary waves pay for NaN checks.
  auto each = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int qw = q0 + j * kBlock + w * 64;
      if (qw >= q1) break;
      const int q = qw + l;
      const bool full = (qw + 64 <= q1) && (qw > 0 || lead == 0) && ((qw + 64) * 4 <= span);
      f(j, q, full);
    }
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
  for (int i = t; i < kBins + 64; i += kBlock) sm.u.hist[i] = 0u;
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
    int blo = 0;  // split tier: bins below blo are merged only if needed
    if (SPLIT) {
      // Bins the row's K-th value can lie in, from the sample alone: the
      // sample holds about lam = K*K/nv scores >= the K-th value, so below
      // the bin where the sample's count from the top reaches lam plus a
      // wide margin the crossing bin is (almost surely) not found.
      // Exactness never depends on this: a row whose count above blo falls
      // short of K merges the remaining bins in a second round.
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const float x = smp[i];
        lds_inc(&sm.u.hist[(x == x) ? vbin(x, gmin, sc) : kBins + l]);
      }
      __syncthreads();
      const float lam = (float)K * (float)K / (float)nv;
      const float rl = lam + 4.0f * sqrtf(lam) + 8.0f;
      const uint32_t rlow = rl >= (float)K ? (uint32_t)K : (uint32_t)rl;
      find_crossing<kBins>([&](int b) { return sm.u.hist[b]; }, rlow, &sm.cross, sm.scan);
      blo = sm.cross.b > 0 ? sm.cross.b : 0;
      for (int i = t; i < kBins + 64; i += kBlock) sm.u.hist[i] = 0u;
      __syncthreads();
    }
    each([&](int j, int q, bool full) {
      if (full) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lds_inc(&sm.u.hist[vbin(v[j][e], gmin, sc)]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = v[j][e];
          lds_inc(&sm.u.hist[(x == x) ? vbin(x, gmin, sc) : kBins + l]);
        }
      }
    });
    __syncthreads();
    if (SPLIT) {
      // publish this workgroup's bins [blo, kBins) densely, then sum the G
      // slices of every bin after the barrier
      uint32_t* mine = s_wh + (size_t)g * kBins;
      for (int b = blo + t; b < kBins; b += kBlock) mine[b] = sm.u.hist[b];
      row_barrier(hdr, G, err);
      auto merged = [&](int b) -> uint32_t {
        uint32_t s = 0;
        for (int gg = 0; gg < G; ++gg) s += s_wh[(size_t)gg * kBins + b];
        return s;
      };
      find_crossing<kBins>([&](int b) { return b >= blo ? merged(b) : 0u; }, (uint32_t)K,
                           &sm.cross, sm.scan);
      if (sm.cross.b < 0 && blo > 0) {
        // the sample's estimate was too high: merge the remaining bins
        for (int b = t; b < blo; b += kBlock) mine[b] = sm.u.hist[b];
        row_barrier(hdr, G, err);
        find_crossing<kBins>(merged, (uint32_t)K, &sm.cross, sm.scan);
      }
    } else {
      find_crossing<kBins>([&](int b) { return sm.u.hist[b]; }, (uint32_t)K, &sm.cross, sm.scan);
    }
    cr = sm.cross;
    path = (cr.b >= 0 && cr.m <= (uint32_t)p.cap) ? 1 : 3;
  }

  if (path == 1) {
    // ---- compaction (a6) --------------------------------------------------
    // bin > b*  <=>  x >= x_hi (winner);  bin == b*  <=>  x_lo <= x < x_hi.
    if (w < 2) {
      const float e = bin_edge(cr.b + w, gmin, sc);
      if (l == 0) sm.thr[w] = e;
    }
    __syncthreads();
    const uint32_t need = (uint32_t)K - cr.above;
    uint32_t wb[NW], cb[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) wb[i] = cb[i] = 0u;
    {
      const float xlo = sm.thr[0], xhi = sm.thr[1];
      each([&](int j, int q, bool) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = j * 4 + e;
          const float x = v[j][e];
          const bool win = x >= xhi;
          const bool cand = (x >= xlo) && !win;
          wb[i >> 5] |= win ? (1u << (i & 31)) : 0u;
          cb[i >> 5] |= cand ? (1u << (i & 31)) : 0u;
        }
      });
    }
    uint32_t nwin = 0, ncand = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      nwin += __popc(wb[i]);
      ncand += __popc(cb[i]);
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
    // winners: walk the set bits (only the index is needed)
    {
      uint32_t wpos = wbase + (ex & 0xFFFFu);
#pragma unroll
      for (int d = 0; d < NW; ++d) {
        uint32_t bits = wb[d];
        while (bits) {
          const int i = d * 32 + __builtin_ctz(bits);
          bits &= bits - 1u;
          const int q = q0 + t + (i >> 2) * kBlock;
          if (wpos < (uint32_t)K) out[wpos] = (q << 2) + (i & 3) - lead;
          ++wpos;
        }
      }
    }
    // candidates: few, so whole waves skip groups without any
    {
      uint32_t cpos = cbase + (ex >> 16);
      const uint32_t ccap = SPLIT ? (uint32_t)kSplitCapMax : (uint32_t)kSingleCap;
      each([&](int j, int q, bool) {
        const uint32_t cq = (cb[(j * 4) >> 5] >> ((j * 4) & 31)) & 0xFu;
        if (__any(cq != 0u)) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool c = (cq >> e) & 1u;
            if (c && cpos < ccap) {
              const uint32_t key = fkey(v[j][e]);
              const int32_t idx = (q << 2) + e - lead;
              if (SPLIT) {
                s_key[cpos] = key;
                s_idx[cpos] = idx;
              } else {
                sm.u.c.key[cpos] = key;
                sm.u.c.idx[cpos] = idx;
              }
            }
            cpos += c ? 1u : 0u;
          }
        }
      });
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
      if (need == m) {
        for (uint32_t i = t; i < m; i += kBlock) out[cr.above + i] = idxs[i];
      } else if (m <= (uint32_t)kRankMax) {
        // Rank counting: candidate i's rank is the number of candidates with
        // a larger key, or an equal key and a smaller index.  Ranks below
        // `need` are selected and written in rank order (value descending,
        // smallest index first inside a tie).
        if (SPLIT) {
          if ((uint32_t)t < m) {
            sm.u.c.key[t] = keys[t];
            sm.u.c.idx[t] = idxs[t];
          }
          __syncthreads();
        }
        if ((uint32_t)t < m) {
          const uint32_t kk = sm.u.c.key[t];
          const int32_t ii = sm.u.c.idx[t];
          uint32_t rank = 0;
          for (uint32_t j = 0; j < m; ++j) {
            const uint32_t kj = sm.u.c.key[j];
            const int32_t ij = sm.u.c.idx[j];
            rank += (kj > kk || (kj == kk && ij < ii)) ? 1u : 0u;
          }
          if (rank < need) out[cr.above + rank] = ii;
        }
      } else {
        // exact radix select of the `need` largest keys among m candidates
        constexpr int CPT = (SPLIT ? kSplitCapMax : kSingleCap) / kBlock;
        uint32_t prefix = 0, rem = need;
        int shift = 24;
        for (int L = 0; L < 4; ++L) {
          shift = 24 - 8 * L;
          sm.dh[t] = 0u;
          __syncthreads();
          for (uint32_t i = t; i < m; i += kBlock) {
            const uint32_t key = keys[i];
            if (L == 0 || ((key ^ prefix) >> (shift + 8)) == 0u)
              lds_inc(&sm.dh[(key >> shift) & 255u]);
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
#pragma unroll
        for (int k2 = 0; k2 < CPT; ++k2) {
          const uint32_t i = t + (uint32_t)k2 * kBlock;
          if (i < m) {
            const uint32_t d = keys[i] >> shift;
            gtm |= (d > thr) ? (1ull << k2) : 0ull;
            eqm |= (d == thr) ? (1ull << k2) : 0ull;
          }
        }
        const uint32_t ngt = (uint32_t)__popcll(gtm), neq = (uint32_t)__popcll(eqm);
        uint32_t tot2;
        const uint32_t ex2 = block_excl_scan((neq << 16) | ngt, sm.scan, tot2);
        uint32_t gpos = cr.above + (ex2 & 0xFFFFu);
        uint32_t tk = ex2 >> 16;
        const uint32_t eqbase = cr.above + (need - rem);
#pragma unroll
        for (int k2 = 0; k2 < CPT; ++k2) {
          const uint32_t i = t + (uint32_t)k2 * kBlock;
          const bool gt = (gtm >> k2) & 1ull;
          const bool eq = (eqm >> k2) & 1ull;
          if (gt && gpos < (uint32_t)K) out[gpos] = idxs[i];
          if (eq && tk < rem) out[eqbase + tk] = idxs[i];
          gpos += gt ? 1u : 0u;
          tk += eq ? 1u : 0u;
        }
      }
    }
    if (SPLIT && refine_here) {
      // last workgroup: put the slot's counters back at rest
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
      each([&](int j, int q, bool) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = rkey(v[j][e]);
          if (L == 0 || ((key ^ prefix) >> (shift + 8)) == 0u)
            lds_inc(&sm.dh[(key >> shift) & 255u]);
        }
      });
      __syncthreads();
      if (SPLIT) {
        // publish this workgroup's digit counts densely; sum the G slices
        s_wd[((size_t)g * 4 + L) * 256 + t] = sm.dh[t];
        row_barrier(hdr, G, err);
        find_crossing<256>(
            [&](int d) {
              uint32_t s = 0;
              for (int gg = 0; gg < G; ++gg) s += s_wd[((size_t)gg * 4 + L) * 256 + d];
              return s;
            },
            rem, &sm.cross, sm.scan);
      } else {
        find_crossing<256>([&](int d) { return sm.dh[d]; }, rem, &sm.cross, sm.scan);
      }
      const Cross c = sm.cross;
      prefix |= (uint32_t)c.b << shift;
      rem -= c.above;
      if (c.m == rem) break;
    }
    const uint32_t thr = prefix >> shift;
    uint32_t ngt = 0, neq = 0;
    each([&](int j, int q, bool) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t d = rkey(v[j][e]) >> shift;
        ngt += (d > thr) ? 1u : 0u;
        neq += (d == thr) ? 1u : 0u;
      }
    });
    if (t == 0) sm.bc[3] = thr;
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
    // re-read after the scan's barriers so the counting pass's compares are
    // not kept live across it
    const uint32_t thr2 = sm.bc[3];
    each([&](int j, int q, bool) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t d = rkey(v[j][e]) >> shift;
        const bool gt = d > thr2;
        const bool eq = d == thr2;
        const int32_t idx = (q << 2) + e - lead;
        if (gt && gpos < (uint32_t)K) out[gpos] = idx;
        if (eq && tk < rem) out[eqbase + tk] = idx;
        gpos += gt ? 1u : 0u;
        tk += eq ? 1u : 0u;
      }
    });
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
