// blockskip.hip -- the block-skip pass of the exact per-row top-K.
//
// The TensorRT-LLM page "Block-skip fast path for self-sampling GVR top-K
// decode" (PR 18122, "Description" and its block-skip commit) adds a row pass
// that reads a side tensor of per-32-score block maxima (bmax) and visits only
// the blocks whose maximum can reach the sampled threshold, falling back to a
// walk over every block when the survivor list overflows; emission, verify
// and the retry ladder stay those of the baseline pass, so the result is the
// same exact selection.  Here, on gfx950, one workgroup (16 waves) owns a
// row:
//  1. guess: the maxima themselves give the floor.  The K largest block maxima
//     are K distinct scores, so the K-th largest of them is at most the row's
//     K-th value: a histogram of the maxima finds a bin edge f below it, and
//     no sample is needed (the pages' pass uses the sampled threshold; with
//     the maxima at hand their order statistic is a floor that exact maxima
//     never put above the K-th value);
//  2. survivors: block i (scores 32i .. 32i+31 of the window) survives unless
//     bmax[i] < f; the survivor ids go to an LDS list (over kBskCap of them:
//     every block);
//  3. verify: a walk over the listed blocks (each wave reads 8 blocks per
//     load, 8 lanes x 16 bytes per block, four loads in flight) counts the
//     scores >= f in an LDS histogram of [f, highest maximum]; the crossing
//     bin b* follows;
//  4. compaction: a second walk writes the scores above b* to the output and
//     keeps b*'s members in LDS; the refine picks the last ones exactly;
//  5. retry ladder: counts short of K (loose bounds put the floor above the
//     K-th value) recount every block with no floor; a crossing bin over the
//     member cap, an invalid bracket or a forced rescue select inside the
//     crossing region (the whole row for the last two) with a radix select
//     whose levels each walk the listed blocks again.
// A block whose maximum is NaN survives (NaN < f is false), so a poisoned pad
// never hides the valid scores of a window's last block.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gvr_common.h"
#include "gvr_device.h"
#include "row_window.h"

namespace ert {

namespace {

constexpr int kBskBlock = 1024;   // threads per row
constexpr int kBskCap = kBskMaxBlocks;  // survivor list / maxima capacity (blocks)
constexpr int kBskMembers = 2048; // crossing-bin members kept in LDS

template <bool SELF>
struct alignas(16) BskSmem {
  uint32_t hist[kBins + 64];  // + one trash word per lane
  float bm[SELF ? kBskCap : 1];  // block maxima made by the first pass
  uint32_t list[kBskCap];     // survivor block ids
  uint32_t key[kBskMembers];
  int32_t idx[kBskMembers];
  alignas(16) uint32_t dh[256];  // radix digit counts (cleared as 16-byte words)
  uint32_t mm[2 * (kBskBlock / 64)];  // per-wave class extremes of a radix level
  uint32_t scan[kBskBlock / 64];
  float rmin[kBskBlock / 64];
  float rmax[kBskBlock / 64];
  Cross cross;
  float thr[2];
  uint32_t ctr[8];
};

}  // namespace

template <int K, bool SELF>
__global__ void __launch_bounds__(kBskBlock) topk_blockskip_kernel(const GvrParams p,
                                                                   const float* bmax,
                                                                   int64_t bmax_stride) {
  constexpr int BLOCK = kBskBlock;
  constexpr int W = BLOCK / 64;
  __shared__ BskSmem<SELF> sm;

  const int t = threadIdx.x;
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t row = (int64_t)p.row_begin + blockIdx.x;
  if (blockIdx.x >= (unsigned)p.rows) return;
  const int S = (int)p.row_stride;
  int ks, nv;
  row_window(p.n_valid, p.row_starts, p.row_ends, p.varlen, row, S, &ks, &nv);
  int32_t* out = p.indices + row * K;
  int32_t* stats = p.row_stats ? p.row_stats + row * kStatsWords : nullptr;

  // ---- short row: identity then -1 ----------------------------------------
  if (nv <= K) {
    for (int i = t; i < K; i += BLOCK) store_nt(out + i, (i < nv) ? i : -1);
    if (stats && t < kStatsWords) stats[t] = (t == 0) ? 0 : (t == 6 ? 1 : (t == 7 ? kBskMembers : -1));
    return;
  }
  const float* win = p.logits + row * (int64_t)S + ks;
  const float* bm_row = SELF ? sm.bm : bmax + row * bmax_stride;
  const int nb = (nv + 31) >> 5;  // blocks of the window
  const float qnan = __builtin_nanf("");

  const f4* win4 = reinterpret_cast<const f4*>(win);
  // Raw buffer over the window's float4 groups: a group past the window reads
  // zeros without a memory access, so every load below is issued
  // unconditionally and the waits for them are exact counts (loads under a
  // lane condition would be waited for one by one).
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(win4, ((nv + 3) & ~3) * 4);
  if (SELF) {
    // ---- first pass: every block once, its maximum kept in LDS -----------
    // (streaming rows of up to kBskCap blocks; U loads in flight per lane)
    constexpr int U = 8;
    const int sub = l & 7;
    for (int s0 = w * 8; s0 < nb; s0 += W * 8 * U) {
      f4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sb = s0 + u * W * 8 + (l >> 3);
        const int q = sb * 32 + sub * 4;  // (q >= nv: out of the buffer's range)
        x[u] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(wrs, q * 4, 0,
                                                                             kCachePolicyNT));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sb = s0 + u * W * 8 + (l >> 3);
        const int q = sb * 32 + sub * 4;
        float m = -__builtin_inff();
#pragma unroll
        for (int e = 0; e < 4; ++e) m = (q + e < nv) ? fmaxf(m, x[u][e]) : m;
        // maximum over the block's 8 lanes
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        if (sub == 0 && sb < nb) sm.bm[sb] = m;
      }
    }
    __syncthreads();
  }

  // ---- guess from the block maxima ----------------------------------------
  // The K largest block maxima are K distinct scores of the row, so the K-th
  // largest of them is at most the row's K-th value: with exact maxima it is
  // a floor that cannot lie above that value, and no sample is needed.  A
  // histogram of the maxima over their finite range finds a bin edge at or
  // below it.  NaN and +inf maxima (loose bounds) count in the top bin.  A
  // window's last, partial block is left out of these statistics and always
  // visited: its maximum may come from the pad past the window (a producer
  // that maximises over the padded row sees the pad's values).
  const int nbf = nv >> 5;  // whole blocks of the window
  for (int i = t; i < kBins + 64; i += BLOCK) sm.hist[i] = 0u;
  if (t < 8) sm.ctr[t] = 0u;
  {
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int i = t; i < nbf; i += BLOCK) {
      const float m = bm_row[i];
      if (__builtin_isfinite(m)) {
        lo = fminf(lo, m);
        hi = fmaxf(hi, m);
      }
    }
    wave_minmax(lo, hi);
    if (l == 0) {
      sm.rmin[w] = lo;
      sm.rmax[w] = hi;
    }
  }
  __syncthreads();
  float bmin = sm.rmin[0], btop = sm.rmax[0];
#pragma unroll
  for (int i = 1; i < W; ++i) {
    bmin = fminf(bmin, sm.rmin[i]);
    btop = fmaxf(btop, sm.rmax[i]);
  }
  bmin = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bmin)));
  btop = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(btop)));
  auto make_map = [](float a, float b, BinMap& m) { return m.set(a, b); };
  float xf = -__builtin_inff();
  bool crowd = false;
  {
    BinMap mm;
    if (make_map(bmin, btop, mm) && nbf >= K && !p.force_rescue) {
      for (int i = t; i < nbf; i += BLOCK) {
        const float m = bm_row[i];
        lds_inc(hword(sm.hist, (m == m) ? vbin_off(m, mm) : 4u * (uint32_t)(kBins - 1)));
      }
      __syncthreads();
      find_crossing<kBins, BLOCK>([&](int b) { return sm.hist[b]; }, (uint32_t)K, &sm.cross,
                                  sm.scan);
      const Cross c = read_cross(&sm.cross);
      if (c.b >= 0) {
        // many equal maxima at or above the floor: aggregate the increments
        for (int i = c.b + t; i < kBins; i += BLOCK)
          if (sm.hist[i] >= 32u) sm.ctr[7] = 1u;
        if (w == 0) {
          const float e = bin_edge(c.b, mm);
          if (l == 0) sm.thr[0] = e;
        }
        __syncthreads();
        xf = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.thr[0])));
        crowd = sm.ctr[7] != 0u;
      }
      __syncthreads();
      for (int i = t; i < kBins + 64; i += BLOCK) sm.hist[i] = 0u;
    }
  }
  // The scores' bracket: [floor, highest maximum].  A row with no floor
  // (fewer than K whole blocks, or unusable maxima) brackets with the block64
  // sample of the other kernel instead (PR 20998 "What changes": K scores in
  // K/64 blocks of 64 spread over the window, both ends included).
  auto sample_bracket = [&](float& lo_out, float& hi_out) {
    constexpr int NSB = K / 64;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int j = w; j < NSB; j += W) {
      const float x = win[SampleStep<NSB>(nv).start(j) + l];
      lo = fminf(lo, x);
      hi = fmaxf(hi, x);
    }
    wave_minmax(lo, hi);
    if (l == 0) {
      sm.rmin[w] = lo;
      sm.rmax[w] = hi;
    }
    __syncthreads();
    lo = sm.rmin[0];
    hi = sm.rmax[0];
#pragma unroll
    for (int i = 1; i < W; ++i) {
      lo = fminf(lo, sm.rmin[i]);
      hi = fmaxf(hi, sm.rmax[i]);
    }
    lo_out = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lo)));
    hi_out = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(hi)));
    __syncthreads();
  };
  float gmin = xf, gmax = btop;
  if (!(xf > -__builtin_inff())) sample_bracket(gmin, gmax);
  BinMap bm;
  bool bracket_ok = make_map(gmin, gmax, bm) && !p.force_rescue;

  // ---- survivors -----------------------------------------------------------
  // nlist == -1: walk every block of the window.
  int nlist = -1;
  if (bracket_ok && xf > -__builtin_inff()) {
    for (int i0 = 0; i0 < nb; i0 += BLOCK) {
      const int i = i0 + t;
      bool keep = false;
      if (i < nb) keep = i >= nbf || !(bm_row[i] < xf);
      const uint32_t pos = wave_append(keep, &sm.ctr[0]);
      if (keep && pos < (uint32_t)kBskCap) sm.list[pos] = (uint32_t)i;
    }
    __syncthreads();
    const uint32_t ns = __builtin_amdgcn_readfirstlane(sm.ctr[0]);
    nlist = ns <= (uint32_t)kBskCap ? (int)ns : -1;
  }

  // Walk the listed blocks: f(x, pos) for every in-window score.  A wave
  // reads 8 blocks per step, lane l taking 16 bytes (l & 7) of block (l >> 3).
  // Decode windows start at the row's 16-byte aligned base and the stride is
  // a multiple of 4, so a group that starts inside the window lies inside the
  // row; lanes past the window's end take no score.
  auto walk = [&](auto&& f) {
    constexpr int U = 4;  // steps whose loads are in flight together
    const int nwalk = nlist < 0 ? nb : nlist;
    const int sub = l & 7;
    for (int s0 = w * 8; s0 < nwalk; s0 += W * 8 * U) {
      f4 x[U];
      int p0[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = s0 + u * W * 8 + (l >> 3);
        p0[u] = -1;
        if (s < nwalk) {
          const int b = nlist < 0 ? s : (int)sm.list[s];
          const int q = b * 32 + sub * 4;
          if (q < nv) p0[u] = q;
        }
        // (no block, or past the window: an offset out of the buffer's range)
        const int off = p0[u] >= 0 ? p0[u] * 4 : ((nv + 3) & ~3) * 4;
        x[u] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0));
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (p0[u] >= 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (p0[u] + e < nv) f(x[u][e], p0[u] + e);
        }
    }
  };

  // ---- verify --------------------------------------------------------------
  int path = 2;  // 1 fast, 2 rescue (invalid bracket), 3 crowded crossing, 5 recount
  Cross cr{-1, 0u, 0u, 0u};
  auto count = [&]() {
    if (crowd) {
      walk([&](float x, int) {
        const bool in = x >= xf;
        lds_inc_agg(sm.hist, in ? (uint32_t)vbin(x, bm) : 0u, in);
      });
    } else {
      walk([&](float x, int) {
        if (x >= xf) lds_inc(hword(sm.hist, vbin_off(x, bm)));
      });
    }
    __syncthreads();
    find_crossing<kBins, BLOCK>([&](int b) { return sm.hist[b]; }, (uint32_t)K, &sm.cross,
                                sm.scan);
    cr = read_cross(&sm.cross);
  };
  if (bracket_ok) {
    count();
    path = 1;
    if (cr.b < 0) {
      // the floor lay above the K-th value (loose maxima): count every block
      // with no floor, in the sample's bracket
      for (int i = t; i < kBins + 64; i += BLOCK) sm.hist[i] = 0u;
      xf = -__builtin_inff();
      nlist = -1;
      sample_bracket(gmin, gmax);
      bracket_ok = make_map(gmin, gmax, bm);
      path = 5;
      if (bracket_ok) count();
    }
    // no crossing even so (NaN scores, outside the contract): the whole row
    if (cr.b < 0) path = 2;
    else if (cr.m > (uint32_t)kBskMembers) path = 3;
  }

  // ---- compaction and refine ----------------------------------------------
  uint32_t nbar = 0;
  if (path == 1 || path == 5) {
    if (w < 2) {
      const float e = bin_edge(cr.b + w, bm);
      if (l == 0) sm.thr[w] = e;
    }
    if (t < 4) sm.ctr[t] = 0u;
    __syncthreads();
    const float xlo = fmaxf(sm.thr[0], xf), xhi = sm.thr[1];
    walk([&](float x, int pos) {
      const bool win_ = x >= xhi;
      const bool mem = !win_ && x >= xlo;
      const uint32_t wp = wave_append(win_, &sm.ctr[0]);
      if (win_ && wp < (uint32_t)K) store_nt(out + wp, pos);
      const uint32_t mp = wave_append(mem, &sm.ctr[1]);
      if (mem && mp < (uint32_t)kBskMembers) {
        sm.key[mp] = fkey(x);
        sm.idx[mp] = pos;
      }
    });
    __syncthreads();
    const uint32_t m = cr.m, need = (uint32_t)K - cr.above;
    if (need == m) {
      for (uint32_t i = t; i < m; i += BLOCK) store_nt(out + cr.above + i, sm.idx[i]);
    } else if (m <= (uint32_t)kRankMax) {
      rank_select_direct<BLOCK>(sm.key, sm.idx, m, need, out, cr.above);
    } else {
      if (t < 2) sm.ctr[t] = 0u;
      __syncthreads();
      list_select<BLOCK>(sm.key, sm.idx, m, need, p.deterministic != 0, out, cr.above, (uint32_t)K,
                         sm.dh, &sm.cross, sm.scan, sm.mm, sm.ctr, nbar);
    }
  } else {
    // ---- radix select inside the crossing region (or the whole row) -------
    float xlo = -__builtin_inff(), xhi = __builtin_inff();
    uint32_t above = 0u;
    bool whole = true;
    if (path == 3) {
      if (w < 2) {
        const float e = bin_edge(cr.b + w, bm);
        if (l == 0) sm.thr[w] = e;
      }
      __syncthreads();
      xlo = fmaxf(sm.thr[0], xf);
      xhi = sm.thr[1];
      above = cr.above;
      whole = false;
    }
    // class: scores in [xlo, xhi) (all scores, NaN included, for the whole
    // row); xhi is NaN when b* is the top bin, which bounds nothing
    auto in_class = [&](float x) { return whole || (x >= xlo && !(x >= xhi)); };
    auto iter = [&](auto&& f) {
      walk([&](float x, int) {
        if (in_class(x)) f(rkey(x));
      });
    };
    const uint32_t need = (uint32_t)K - above;
    // (aggregated increments and the single-key stop: tie-heavy rows that
    // reach this path, e.g. an all-equal row whose maxima all equal the
    // floor, otherwise pay 64-way LDS conflicts on one digit at every level)
    const RSel s = radix_select<BLOCK, true, true>(iter, need, sm.dh, &sm.cross, sm.scan, sm.mm,
                                                   nullptr, nullptr, nullptr, 1, nbar, BarrierSync{});
    const bool pick = p.deterministic && s.cnt > s.rem;
    RSel s2{0u, 0, 0u, 0u};
    if (pick) {
      const uint32_t tk = s.thr;  // the select ended on one exact key
      s2 = radix_select<BLOCK, true, true>(
          [&](auto&& f) {
            walk([&](float x, int pos) {
              if (in_class(x)) f(rkey(x) == tk ? ~(uint32_t)pos : 0u);
            });
          },
          s.rem, sm.dh, &sm.cross, sm.scan, sm.mm, nullptr, nullptr, nullptr, 1, nbar, BarrierSync{});
    }
    if (t < 4) sm.ctr[t] = 0u;
    __syncthreads();
    const uint32_t eqbase = (uint32_t)K - s.rem;
    walk([&](float x, int pos) {
      bool gt = !whole && x >= xhi;
      bool eq = false;
      if (in_class(x)) {
        const uint32_t d = rkey(x) >> s.shift;
        gt = d > s.thr;
        eq = d == s.thr && (!pick || ((~(uint32_t)pos) >> s2.shift) >= s2.thr);
      }
      const uint32_t gp = wave_append(gt, &sm.ctr[0]);
      if (gt && gp < eqbase) store_nt(out + gp, pos);
      const uint32_t tk = wave_append(eq, &sm.ctr[1]);
      if (eq && tk < s.rem) store_nt(out + eqbase + tk, pos);
    });
  }
  if (stats && t == 0) {
    stats[0] = path;
    stats[1] = bracket_ok ? (int)cr.m : -1;
    stats[2] = bracket_ok ? (int)cr.above : -1;
    stats[3] = bracket_ok ? cr.b : -1;
    stats[4] = (int)__float_as_uint(gmin);
    stats[5] = (int)__float_as_uint(gmax);
    stats[6] = 1;
    stats[7] = kBskMembers;
    stats[8] = nlist < 0 ? nb : nlist;  // blocks the last walk visited
  }
}

__global__ void __launch_bounds__(256) block_max_kernel(const float* logits, int64_t row_stride,
                                                        int32_t num_rows, float* bmax,
                                                        int64_t bmax_stride) {
  // one thread per block of 32: bmax[r][i] = max over logits[r][32i .. 32i+31]
  // (NaN-ignoring; a block of NaN only gives NaN)
  const int64_t nb = (row_stride + 31) / 32;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = gid / nb, i = gid - r * nb;
  if (r >= num_rows) return;
  const float* x = logits + r * row_stride + i * 32;
  const int n = (int)((row_stride - i * 32) < 32 ? (row_stride - i * 32) : 32);
  float m = __builtin_nanf("");
  for (int e = 0; e < n; ++e) m = fmaxf(m, x[e]);
  bmax[r * bmax_stride + i] = m;
}

const void* blockskip_kernel(int k, bool self) {
  switch (k) {
    case 512:
      return self ? reinterpret_cast<const void*>(&topk_blockskip_kernel<512, true>)
                  : reinterpret_cast<const void*>(&topk_blockskip_kernel<512, false>);
    case 1024:
      return self ? reinterpret_cast<const void*>(&topk_blockskip_kernel<1024, true>)
                  : reinterpret_cast<const void*>(&topk_blockskip_kernel<1024, false>);
    case 2048:
      return self ? reinterpret_cast<const void*>(&topk_blockskip_kernel<2048, true>)
                  : reinterpret_cast<const void*>(&topk_blockskip_kernel<2048, false>);
    default: return nullptr;
  }
}

// The same maxima with coalesced loads (16-byte aligned rows of a multiple of
// 4 floats): eight lanes per block of 32, one 16-byte load each, so a wave
// reads 1 KiB of consecutive scores per load; a 3-step exchange finds each
// block's maximum.
__global__ void __launch_bounds__(256) block_max_vec_kernel(const float* logits, int64_t row_stride,
                                                            int32_t num_rows, float* bmax,
                                                            int64_t bmax_stride) {
  const int64_t nb = (row_stride + 31) / 32;
  const int64_t gb = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;  // this lane's block
  const int sub = (int)(threadIdx.x & 7u);
  const int64_t r = gb / nb, i = gb - r * nb;
  float m = __builtin_nanf("");
  if (r < num_rows) {
    const int64_t col = i * 32 + sub * 4;
    if (col < row_stride) {  // (row_stride % 4 == 0: the whole float4 lies in the row)
      const f4 x = *reinterpret_cast<const f4*>(logits + r * row_stride + col);
      m = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    }
  }
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  m = fmaxf(m, __shfl_xor(m, 4, 64));
  if (r < num_rows && sub == 0) bmax[r * bmax_stride + i] = m;
}

const void* block_max_kernel_ptr(bool vec) {
  return vec ? reinterpret_cast<const void*>(&block_max_vec_kernel)
             : reinterpret_cast<const void*>(&block_max_kernel);
}

}  // namespace ert
