// gvr_device.h -- device helpers shared by the selection kernels: the
// order-preserving key, the value-histogram bin map and its bin edges, LDS
// and wave primitives, the crossing-bin search, the row barrier of the split
// tier, and the exact refine / radix selection over a set of keys.
#ifndef ERT_GVR_DEVICE_H_
#define ERT_GVR_DEVICE_H_

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

// Raw buffer resource, word 3 for gfx9-family parts (32-bit data format,
// no swizzle); loads past num_records return zeros without a memory access.
constexpr int kBufWord3 = 0x00020000;
// Cache policy of streaming loads: non-temporal (the scores are read once).
constexpr int kCachePolicyNT = 2;
// Cache policy of stores that other workgroups read by agent-scope atomic
// loads: sc1, as on the compiler's own agent-scope atomic stores.
constexpr int kCachePolicyAgent = 16;

// Raw buffer resource over [p, p + bytes) (p and bytes uniform: both go
// through readfirstlane so the descriptor lives in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, __builtin_amdgcn_readfirstlane(bytes),
                                           kBufWord3);
}

// Start of block j of the block64 sample over a window of nv > 64 * NSB scores:
// floor(j * (nv - 64) / (NSB - 1)).  With nv - 64 = a (NSB - 1) + b, 0 <= b <
// NSB - 1, that is j a + floor(j b / (NSB - 1)) exactly, so one 32-bit quotient
// and remainder per row replace a 64-bit division per block (j b < 32 * 32).
template <int NSB>
struct SampleStep {
  uint32_t a, b;
  __device__ __forceinline__ explicit SampleStep(int nv)
      : a((uint32_t)(nv - 64) / (uint32_t)(NSB - 1)), b((uint32_t)(nv - 64) % (uint32_t)(NSB - 1)) {}
  __device__ __forceinline__ int start(int j) const {
    return (int)((uint32_t)j * a + ((uint32_t)j * b) / (uint32_t)(NSB - 1));
  }
};

// A float pinned to a scalar register: as an operand of a VOP3 instruction it
// takes the one scalar slot instead of a literal the compiler would otherwise
// rematerialise into a VGPR before every use.
__device__ __forceinline__ float sgpr_f32(float x) {
  asm("" : "+s"(x));
  return x;
}

// The bracket's bin map over [lo, hi]: with sc4 = 4 kBins / (hi - lo) and
// cm = 2^23 - lo * sc4 (each rounded once per row), t = fma(x, sc4, cm)
// clamped to [2^23, 2^23 + 4 (kBins - 1)] is a float whose unit in the last
// place is 1, so t is a whole number and its low 23 bits are t - 2^23: bin(x)
// is that number divided by 4 and rounded down, and the bin's LDS byte offset
// is the same bits with the low two cleared -- one mask, no float-to-integer
// conversion.  The fused multiply-add, the clamp and the mask are each
// monotone non-decreasing in x, so equal values share a bin and bins ascend
// with the value; this is the single definition every step uses.  Folding
// 2^23 into the addend shifts the partition by at most half a unit of cm: a
// fraction of a bin unless the bracket is narrower than about 1e-6 of its
// magnitude, where bins merge (the selection stays exact; a crowded bin takes
// the rescue).  The mask also keeps a NaN's index in range (NaN scores are
// outside the contract).
struct BinMap {
  float gmin, sc, sc4, cm;
  float lo23 = sgpr_f32(8388608.0f);                        // 2^23
  float hi23 = sgpr_f32(8388608.0f + 4.0f * (kBins - 1));  // 2^23 + the top bin's offset
  // the map of [lo, hi] (both uniform); false when the bracket cannot carry one
  __device__ __forceinline__ bool set(float lo, float hi) {
    const float range = hi - lo;
    gmin = lo;
    sc = (float)kBins / range;
    // (uniform: scalar registers, which the histogram passes copy into a
    // vector register where an instruction needs one, rather than holding a
    // vector register for them across the row)
    sc4 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(4.0f * sc)));
    cm = __int_as_float(
        __builtin_amdgcn_readfirstlane(__float_as_int(__builtin_fmaf(-lo, sc4, 8388608.0f))));
    return __builtin_isfinite(lo) && __builtin_isfinite(hi) && (hi > lo) &&
           __builtin_isfinite(range) && __builtin_isfinite(sc4) && __builtin_isfinite(cm) &&
           (sc > 0.0f);
  }
};
__device__ __forceinline__ uint32_t vbin_off(float x, const BinMap& bm) {
  float t = __builtin_fmaf(x, bm.sc4, bm.cm);
  t = __builtin_amdgcn_fmed3f(t, bm.lo23, bm.hi23);
  return __float_as_uint(t) & (uint32_t)(4 * kBins - 4);
}
__device__ __forceinline__ int vbin(float x, const BinMap& bm) { return (int)(vbin_off(x, bm) >> 2); }
// Output indices are written once and never read again by the selection:
// non-temporal stores stream them past the caches (on the 4096 x 16640
// prefill tile about 2 % faster than plain stores).
__device__ __forceinline__ void store_nt(int32_t* p, int32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt4(int32_t* p, const int32_t* src) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(src), reinterpret_cast<v4i*>(p));
}

// The winner walk: a thread's bit word d (groups 8 d .. 8 d + 7 of the
// thread, first score in the highest of nb bits) is shifted left by 32 - nb
// so that the leading-zero count c of a set bit is the score's place in the
// word: lane c % 4 of group 8 d + c / 4.  Groups of one thread lie 4 BLOCK
// scores apart, which is c's bits 2..4 shifted up by log2(BLOCK): both
// fields come from one shift-or and one mask.
template <int BLOCK>
__device__ __forceinline__ int walk_offset(uint32_t c) {
  static_assert(BLOCK == 256 || BLOCK == 512 || BLOCK == 1024, "power-of-two workgroups");
  constexpr uint32_t kLog = BLOCK == 256 ? 8u : BLOCK == 512 ? 9u : 10u;
  return (int)(((c << kLog) | c) & ((0x1Cu << kLog) | 3u));
}
// Pop the first set bit of a left-aligned walk word: its leading-zero count.
__device__ __forceinline__ uint32_t walk_pop(uint32_t& bits) {
  const uint32_t c = (uint32_t)__builtin_clz(bits);
  bits ^= 0x80000000u >> c;
  // (the loop then tests the cleared word itself, not the old one against
  // the bit, which would keep both live)
  asm volatile("" : "+v"(bits));
  return c;
}

// One lane's float4 group against the crossing bin's edges [xlo, xhi) (both
// uniform): its four winner bits (x >= xhi) are shifted into wacc and its
// four member bits (xlo <= x < xhi) into cacc, each by add-with-carry
// doublings (acc = 2 acc + bit: the group's first score lands in the highest
// of the four new bits).  NaN compares false both ways.  Every scalar pair a
// doubling reads as its carry-in was written four or more instructions
// earlier.  The member masks come from scalar and-nots inside the block,
// which write SCC: declared clobbered, so no compare the compiler made
// before the block is read after it.  Compared with a compare and a select
// per bit, this takes two VALU instructions per score and threshold and no
// wait states.
__device__ __forceinline__ void group_bits(const f4& x, float xlo, float xhi, uint32_t& wacc,
                                           uint32_t& cacc) {
  uint64_t h0, h1, h2, h3, g0, g1, g2, g3, cy;
  asm("v_cmp_ge_f32_e64 %[h0], %[x0], %[hi]\n\t"
      "v_cmp_ge_f32_e64 %[h1], %[x1], %[hi]\n\t"
      "v_cmp_ge_f32_e64 %[h2], %[x2], %[hi]\n\t"
      "v_cmp_ge_f32_e64 %[h3], %[x3], %[hi]\n\t"
      "v_cmp_ge_f32_e64 %[g0], %[x0], %[lo]\n\t"
      "v_cmp_ge_f32_e64 %[g1], %[x1], %[lo]\n\t"
      "v_cmp_ge_f32_e64 %[g2], %[x2], %[lo]\n\t"
      "v_cmp_ge_f32_e64 %[g3], %[x3], %[lo]\n\t"
      "s_andn2_b64 %[g0], %[g0], %[h0]\n\t"
      "s_andn2_b64 %[g1], %[g1], %[h1]\n\t"
      "s_andn2_b64 %[g2], %[g2], %[h2]\n\t"
      "s_andn2_b64 %[g3], %[g3], %[h3]\n\t"
      "v_addc_co_u32_e64 %[w], %[cy], %[w], %[w], %[h0]\n\t"
      "v_addc_co_u32_e64 %[w], %[cy], %[w], %[w], %[h1]\n\t"
      "v_addc_co_u32_e64 %[w], %[cy], %[w], %[w], %[h2]\n\t"
      "v_addc_co_u32_e64 %[w], %[cy], %[w], %[w], %[h3]\n\t"
      "v_addc_co_u32_e64 %[c], %[cy], %[c], %[c], %[g0]\n\t"
      "v_addc_co_u32_e64 %[c], %[cy], %[c], %[c], %[g1]\n\t"
      "v_addc_co_u32_e64 %[c], %[cy], %[c], %[c], %[g2]\n\t"
      "v_addc_co_u32_e64 %[c], %[cy], %[c], %[c], %[g3]"
      : [w] "+v"(wacc), [c] "+v"(cacc), [h0] "=&s"(h0), [h1] "=&s"(h1), [h2] "=&s"(h2),
        [h3] "=&s"(h3), [g0] "=&s"(g0), [g1] "=&s"(g1), [g2] "=&s"(g2), [g3] "=&s"(g3),
        [cy] "=&s"(cy)
      : [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [x3] "v"(x[3]), [hi] "s"(xhi),
        [lo] "s"(xlo)
      : "scc");
}

// The winner bits of group_bits alone, and the member lane masks g[e]
// (xlo <= x[e] < xhi) handed back in scalar registers instead of being
// shifted into a second word: members are rare, so a group with none costs
// three scalar ors and a branch (append_members below takes the others).
__device__ __forceinline__ void group_wins(const f4& x, float xlo, float xhi, uint32_t& wacc,
                                           uint64_t (&g)[4]) {
  uint64_t h0, h1, h2, h3, cy;
  asm("v_cmp_ge_f32_e64 %[h0], %[x0], %[hi]\n\t"
      "v_cmp_ge_f32_e64 %[h1], %[x1], %[hi]\n\t"
      "v_cmp_ge_f32_e64 %[h2], %[x2], %[hi]\n\t"
      "v_cmp_ge_f32_e64 %[h3], %[x3], %[hi]\n\t"
      "v_cmp_ge_f32_e64 %[g0], %[x0], %[lo]\n\t"
      "v_cmp_ge_f32_e64 %[g1], %[x1], %[lo]\n\t"
      "v_cmp_ge_f32_e64 %[g2], %[x2], %[lo]\n\t"
      "v_cmp_ge_f32_e64 %[g3], %[x3], %[lo]\n\t"
      "s_andn2_b64 %[g0], %[g0], %[h0]\n\t"
      "s_andn2_b64 %[g1], %[g1], %[h1]\n\t"
      "s_andn2_b64 %[g2], %[g2], %[h2]\n\t"
      "s_andn2_b64 %[g3], %[g3], %[h3]\n\t"
      "v_addc_co_u32_e64 %[w], %[cy], %[w], %[w], %[h0]\n\t"
      "v_addc_co_u32_e64 %[w], %[cy], %[w], %[w], %[h1]\n\t"
      "v_addc_co_u32_e64 %[w], %[cy], %[w], %[w], %[h2]\n\t"
      "v_addc_co_u32_e64 %[w], %[cy], %[w], %[w], %[h3]"
      : [w] "+v"(wacc), [h0] "=&s"(h0), [h1] "=&s"(h1), [h2] "=&s"(h2), [h3] "=&s"(h3),
        [g0] "=&s"(g[0]), [g1] "=&s"(g[1]), [g2] "=&s"(g[2]), [g3] "=&s"(g[3]), [cy] "=&s"(cy)
      : [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [x3] "v"(x[3]), [hi] "s"(xhi),
        [lo] "s"(xlo)
      : "scc");
}

// LDS histogram word at a byte offset from vbin_off.
__device__ __forceinline__ uint32_t* hword(uint32_t* h, uint32_t off) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(h) + off);
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_add_agent_nr(uint32_t* p, uint32_t v) {
  (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's vector memory operations (stores, atomics) have
// completed: s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt fields at
// their no-wait maxima).  Every wave runs it before the workgroup barrier
// that precedes one thread's release and arrival, so what all waves wrote is
// performed before any other workgroup can see the arrival.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void lds_inc(uint32_t* p) {
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint32_t lds_take(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Count one per lane with `act` into h[d]; when every such lane of the wave
// has the same d (tie-heavy rows), one lane adds them all at once instead of
// 64 conflicting increments.  The first lane's d comes from readfirstlane
// (no LDS round trip).  Must be reached by the whole wave.
__device__ __forceinline__ void lds_inc_agg(uint32_t* h, uint32_t d, bool act) {
  if (act) {
    const uint32_t d0 = __builtin_amdgcn_readfirstlane(d);
    const uint64_t am = __ballot(1);
    const uint64_t same = __ballot(d == d0);
    if (same == am) {
      if ((uint32_t)lane_id() == (uint32_t)(__ffsll((unsigned long long)am) - 1))
        __hip_atomic_fetch_add(&h[d0], (uint32_t)__popcll(am), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      __hip_atomic_fetch_add(&h[d], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
}

// Append the lanes with `pred` to an LDS-counted list: one atomic per wave,
// lane order inside the wave.  Returns each predicated lane's position.
// Must be reached by the whole wave.
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* ctr) {
  const uint64_t m = __ballot(pred);
  uint32_t base = 0;
  if (m != 0ull) {
    const int leader = __ffsll((unsigned long long)m) - 1;
    if (lane_id() == leader)
      base = __hip_atomic_fetch_add(ctr, (uint32_t)__popcll(m), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_WORKGROUP);
    base = __shfl(base, leader, 64);
  }
  const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  return base + below;
}


// The `need` largest of the m (key, index) pairs held in LDS (m small), by
// rank counting: pair i's rank is the number of pairs with a larger key, or
// an equal key and a smaller index, so ties go to the smallest indices.  No
// barrier of its own (the list is complete and visible when it starts): the
// tail of the last group of four is masked by position rather than padded,
// and each pick goes straight to out[base + rank] (global memory), so no
// wave waits for another once the list is built.
template <int BLOCK>
__device__ __forceinline__ void rank_select_direct(const uint32_t* key, const int32_t* idx,
                                                   uint32_t m, uint32_t need, int32_t* out,
                                                   uint32_t base) {
  for (uint32_t i = threadIdx.x; i < m; i += BLOCK) {
    const uint32_t kk = key[i];
    const int32_t ii = idx[i];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < m; j += 4) {
      const uint4 kj = *reinterpret_cast<const uint4*>(key + j);
      const int4 ij = *reinterpret_cast<const int4*>(idx + j);
      rank += (kj.x > kk || (kj.x == kk && ij.x < ii)) ? 1u : 0u;
      rank += (j + 1 < m && (kj.y > kk || (kj.y == kk && ij.y < ii))) ? 1u : 0u;
      rank += (j + 2 < m && (kj.z > kk || (kj.z == kk && ij.z < ii))) ? 1u : 0u;
      rank += (j + 3 < m && (kj.w > kk || (kj.w == kk && ij.w < ii))) ? 1u : 0u;
    }
    if (rank < need) store_nt(out + base + rank, ii);
  }
}

// ---------------------------------------------------------------------------
// Wave and block primitives
// ---------------------------------------------------------------------------

// Workgroup barrier for LDS traffic only: the fences are scoped to LDS, so
// the barrier waits for this wave's LDS operations (lgkmcnt) but not for its
// global loads and stores, which may stay in flight across it (a kernel that
// loads its next row during this one's selection relies on that).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave-wide scans and reductions as in-place DPP-fused instructions: each
// step combines a lane with the lane that its row shift (within rows of 16)
// or row broadcast (lane 15 / 31 into the following rows, row_mask) names.
// Without bound_ctrl a lane whose source lies outside its row is not
// written, which is what a scan (adding nothing) and an idempotent min / max
// want: no lane test and no select per step, one instruction per value.  A
// DPP read of a register that a vector instruction wrote needs two wait
// states on gfx9: the s_nop 1 ahead of every step.  The inputs' own writers
// are covered by the first step's s_nop as well.
#define ERT_DPP_STEP1(OP, R, CTL, RMASK) \
  "s_nop 1\n\t" OP " " R ", " R ", " R " " CTL " row_mask:" RMASK " bank_mask:0xf\n\t"
#define ERT_DPP_STEP2(OPA, OPB, RA, RB, CTL, RMASK)                                  \
  "s_nop 1\n\t" OPA " " RA ", " RA ", " RA " " CTL " row_mask:" RMASK " bank_mask:0xf\n\t" \
  OPB " " RB ", " RB ", " RB " " CTL " row_mask:" RMASK " bank_mask:0xf\n\t"

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts
// (within rows of 16) and the gfx9 row broadcasts (across rows).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  asm(ERT_DPP_STEP1("v_add_u32_dpp", "%0", "row_shr:1", "0xf")
      ERT_DPP_STEP1("v_add_u32_dpp", "%0", "row_shr:2", "0xf")
      ERT_DPP_STEP1("v_add_u32_dpp", "%0", "row_shr:4", "0xf")
      ERT_DPP_STEP1("v_add_u32_dpp", "%0", "row_shr:8", "0xf")
      ERT_DPP_STEP1("v_add_u32_dpp", "%0", "row_bcast:15", "0xa")
      ERT_DPP_STEP1("v_add_u32_dpp", "%0", "row_bcast:31", "0xc")
      : "+v"(v));
  return v;
}

// Min and max over a wave (read from lane 63 into every lane).  A quiet NaN
// (the kernels' markers) is ignored: in IEEE mode v_min / v_max return the
// other operand.
__device__ __forceinline__ void wave_minmax(float& mn, float& mx) {
  asm(ERT_DPP_STEP2("v_min_f32_dpp", "v_max_f32_dpp", "%0", "%1", "row_shr:1", "0xf")
      ERT_DPP_STEP2("v_min_f32_dpp", "v_max_f32_dpp", "%0", "%1", "row_shr:2", "0xf")
      ERT_DPP_STEP2("v_min_f32_dpp", "v_max_f32_dpp", "%0", "%1", "row_shr:4", "0xf")
      ERT_DPP_STEP2("v_min_f32_dpp", "v_max_f32_dpp", "%0", "%1", "row_shr:8", "0xf")
      ERT_DPP_STEP2("v_min_f32_dpp", "v_max_f32_dpp", "%0", "%1", "row_bcast:15", "0xa")
      ERT_DPP_STEP2("v_min_f32_dpp", "v_max_f32_dpp", "%0", "%1", "row_bcast:31", "0xc")
      : "+v"(mn), "+v"(mx));
  mn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mn), 63));
  mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 63));
}

// Largest of a and of b over a wave (result in every lane, from lane 63).
__device__ __forceinline__ void wave_max2_u32(uint32_t& a, uint32_t& b) {
  asm(ERT_DPP_STEP2("v_max_u32_dpp", "v_max_u32_dpp", "%0", "%1", "row_shr:1", "0xf")
      ERT_DPP_STEP2("v_max_u32_dpp", "v_max_u32_dpp", "%0", "%1", "row_shr:2", "0xf")
      ERT_DPP_STEP2("v_max_u32_dpp", "v_max_u32_dpp", "%0", "%1", "row_shr:4", "0xf")
      ERT_DPP_STEP2("v_max_u32_dpp", "v_max_u32_dpp", "%0", "%1", "row_shr:8", "0xf")
      ERT_DPP_STEP2("v_max_u32_dpp", "v_max_u32_dpp", "%0", "%1", "row_bcast:15", "0xa")
      ERT_DPP_STEP2("v_max_u32_dpp", "v_max_u32_dpp", "%0", "%1", "row_bcast:31", "0xc")
      : "+v"(a), "+v"(b));
  a = (uint32_t)__builtin_amdgcn_readlane((int)a, 63);
  b = (uint32_t)__builtin_amdgcn_readlane((int)b, 63);
}

// Exclusive prefix sum over the block in thread order; `total` gets the sum.
// `sm` holds BLOCK/64 words.  Contains two workgroup barriers.
// Exclusive offsets of v over the whole workgroup in an arbitrary wave order:
// a wave prefix sum and one LDS add per wave on *ctr (zero beforehand).  No
// workgroup barrier.  Must be reached by the whole wave.
__device__ __forceinline__ uint32_t wave_offsets(uint32_t v, uint32_t* ctr) {
  const uint32_t inc = wave_incl_scan(v);
  uint32_t base = 0u;
  if (lane_id() == 63)
    base = __hip_atomic_fetch_add(ctr, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, 63);
  return base + inc - v;
}

// One group's members (the lane masks g[e] of group_wins, not all zero; a
// uniform branch) appended to the LDS member list: one workgroup-scope add
// per wave reserves their slots in the high half of *ctr (whose low half
// wave_offsets uses for the winners), then each member lane writes its key
// and position, pos0 + e.  Slots at or past cap are dropped (the row then
// holds more members than the list, which the caller has ruled out).
__device__ __forceinline__ void append_members(const f4& x, int pos0, const uint64_t (&g)[4],
                                               uint32_t* ctr, uint32_t* key, int32_t* idx,
                                               uint32_t cap) {
  uint32_t n[4], tot = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    n[e] = (uint32_t)__popcll(g[e]);
    tot += n[e];
  }
  const int f = __ffsll((unsigned long long)__ballot(1)) - 1;
  uint32_t b = 0u;
  if (lane_id() == f)
    b = __hip_atomic_fetch_add(ctr, tot << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  b = (uint32_t)__builtin_amdgcn_readlane((int)b, f) >> 16;
  const uint32_t l = (uint32_t)lane_id();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if ((g[e] >> l) & 1ull) {
      const uint32_t s = b + __builtin_amdgcn_mbcnt_hi((uint32_t)(g[e] >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)g[e], 0u));
      if (s < cap) {
        key[s] = fkey(x[e]);
        idx[s] = pos0 + e;
      }
    }
    b += n[e];
  }
}

template <int BLOCK>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sm, uint32_t& total) {
  constexpr int W = BLOCK / 64;
  const uint32_t inc = wave_incl_scan(v);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 63) sm[w] = inc;
  lds_sync();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t s = sm[i];
    off += (i < w) ? s : 0u;
    tot += s;
  }
  lds_sync();
  total = tot;
  return off + inc - v;
}

struct Cross {
  int b;           // crossing bin / digit, -1 if the total is below target
  uint32_t above;  // count strictly above it
  uint32_t m;      // count inside it
  uint32_t total;
};

// The crossing that find_crossing left in LDS, held in scalar registers (every
// lane reads the same words; readfirstlane keeps them out of the VGPR budget
// the resident row needs).
__device__ __forceinline__ Cross read_cross(const Cross* c) {
  Cross r;
  r.b = __builtin_amdgcn_readfirstlane(c->b);
  r.above = __builtin_amdgcn_readfirstlane(c->above);
  r.m = __builtin_amdgcn_readfirstlane(c->m);
  r.total = __builtin_amdgcn_readfirstlane(c->total);
  return r;
}

// The crossing from counts already in registers: thread t holds c[i] =
// h[NBINS - 1 - t * PER - i] (PER consecutive bins from the top; threads
// past NBINS / PER hold zeros).  Result in *out (LDS), visible to all threads
// on return.
template <int NBINS, int BLOCK, int PER>
__device__ __forceinline__ void crossing_from(const uint32_t (&c)[PER], uint32_t target, Cross* out,
                                              uint32_t* scan_sm) {
  constexpr int OWNERS = NBINS / PER;
  const int t = threadIdx.x;
  const int hi = NBINS - 1 - t * PER;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += c[i];
  uint32_t tot;
  const uint32_t ex = block_excl_scan<BLOCK>(s, scan_sm, tot);
  if (t < OWNERS && ex < target && ex + s >= target) {
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
  lds_sync();
}

// Find the highest bin b with sum_{b' >= b} h[b'] >= target over NBINS bins,
// where load(b) returns h[b].  Thread t owns PER consecutive bins from the
// top.  Result in *out (LDS), visible to all threads on return.
template <int NBINS, int BLOCK, class Load>
__device__ __forceinline__ void find_crossing(Load&& load, uint32_t target, Cross* out,
                                              uint32_t* scan_sm) {
  constexpr int PER = NBINS >= BLOCK ? NBINS / BLOCK : 1;
  constexpr int OWNERS = NBINS / PER;
  static_assert(PER * OWNERS == NBINS, "bins per thread");
  const int t = threadIdx.x;
  const int hi = NBINS - 1 - t * PER;
  uint32_t c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) c[i] = (t < OWNERS) ? load(hi - i) : 0u;
  crossing_from<NBINS, BLOCK, PER>(c, target, out, scan_sm);
}

// The crossing over the kBins-word LDS histogram h with a single workgroup
// barrier: thread t sums its kBins / BLOCK bins from the top, a wave prefix
// sum plus the waves' totals (through scan_sm, after the barrier) give every
// wave the wave whose bins hold the crossing; each wave then sums that
// wave's per-thread bins again, picks the thread, and 32 or fewer lanes read
// its bins one each to pick the bin.  Every wave returns the same answer in
// scalar registers.  h and scan_sm must not change until every wave is past
// its reads (a writer waits at a workgroup barrier first).
template <int BLOCK>
__device__ __forceinline__ Cross crossing_1sync(const uint32_t* h, uint32_t target,
                                                uint32_t* scan_sm) {
  constexpr int PER = kBins / BLOCK;
  constexpr int W = BLOCK / 64;
  static_assert(PER * BLOCK == kBins && PER <= 64, "bins per thread");
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  auto owner_sum = [&](int owner) {
    const int hi = kBins - 1 - owner * PER;
    uint32_t s = 0u;
#pragma unroll
    for (int i = 0; i < PER; ++i) s += h[hi - i];
    return s;
  };
  const uint32_t s = owner_sum((int)threadIdx.x);
  const uint32_t inc = wave_incl_scan(s);
  if (l == 63) scan_sm[w] = inc;
  lds_sync();
  uint32_t run = 0u, exw = 0u;
  int cw = -1;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t c = (uint32_t)__builtin_amdgcn_readfirstlane((int)scan_sm[i]);
    if (cw < 0 && run + c >= target) {
      cw = i;
      exw = run;
    }
    run += c;
  }
  Cross r;
  r.total = run;
  if (cw < 0) {
    r.b = -1;
    r.above = run;
    r.m = 0u;
    return r;
  }
  const uint32_t s2 = owner_sum(cw * 64 + l);
  const uint32_t inc2 = exw + wave_incl_scan(s2);
  const uint64_t hit = __ballot(inc2 - s2 < target && inc2 >= target);
  const int f = (int)__builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
  const uint32_t ex = (uint32_t)__builtin_amdgcn_readlane((int)(inc2 - s2), f);
  const int hi = kBins - 1 - (cw * 64 + f) * PER;
  const uint32_t c = l < PER ? h[hi - l] : 0u;
  const uint32_t inc3 = ex + wave_incl_scan(c);
  const uint64_t hit2 = __ballot(l < PER && inc3 - c < target && inc3 >= target);
  const int g = (int)__builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit2) - 1);
  r.b = hi - g;
  r.above = (uint32_t)__builtin_amdgcn_readlane((int)(inc3 - c), g);
  r.m = (uint32_t)__builtin_amdgcn_readlane((int)c, g);
  return r;
}

// Smallest score x (IEEE order over [-inf, +inf]) with vbin(x) >= b, so that
// for every non-NaN x: vbin(x) >= b  <=>  x >= edge.  vbin is monotone in x,
// so the set is an up-set.  The 64 lanes first probe the keys around an
// arithmetic estimate of the edge (within an ulp of it for brackets near
// zero); if the edge is not among them, a 64-way search over the keys of
// -inf .. +inf (six rounds) finds it.  b <= 0 gives -inf; b >= kBins gives
// NaN, which no score compares >= to.  Must be called by a whole wave.
__device__ __forceinline__ float bin_edge(int b, const BinMap& bm) {
  if (b <= 0) return -__builtin_inff();
  if (b >= kBins) return __builtin_nanf("");
  uint32_t lo = 0x007FFFFFu;  // key(-inf): vbin = 0 < b
  uint32_t hi = 0xFF800000u;  // key(+inf): vbin = kBins - 1 >= b
  const uint32_t l = (uint32_t)lane_id();
  {
    // bin b starts where fma(x, sc4, cm) rounds to 2^23 + 4 b or more, at
    // x = (2^23 - cm + 4 b - 1/2) / sc4 (2^23 - cm is exact while the
    // bracket's lower end lies within 512 widths of zero; elsewhere the
    // search below finds the edge all the same)
    const float est = ((8388608.0f - bm.cm) + (4.0f * (float)b - 0.5f)) / bm.sc4;
    const uint32_t c = fkey(est);
    const int64_t pk = (int64_t)c - 31 + (int64_t)l;
    const uint32_t probe =
        pk < (int64_t)lo ? lo : (pk > (int64_t)hi ? hi : (uint32_t)pk);
    const bool ok = vbin(from_key(probe), bm) >= b;
    const uint64_t mask = __ballot(ok);
    if (mask != 0ull && (mask & 1ull) == 0ull) {
      // the first passing lane is the edge unless probes were clamped
      const int f = __ffsll((unsigned long long)mask) - 1;
      const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)probe, f);
      const uint32_t below = (uint32_t)__builtin_amdgcn_readlane((int)probe, f - 1);
      if (below + 1u == e) return from_key(e);
      lo = below;
      hi = e;
    } else if (mask == 0ull) {
      lo = (uint32_t)__builtin_amdgcn_readlane((int)probe, 63);
    } else {
      hi = (uint32_t)__builtin_amdgcn_readlane((int)probe, 0);
    }
  }
  while (hi - lo > 1u) {
    const uint32_t span = hi - lo;
    const uint32_t step = span / 64u + ((span & 63u) ? 1u : 0u);
    const uint64_t pk = (uint64_t)lo + (uint64_t)(l + 1u) * step;
    const uint32_t probe = pk >= (uint64_t)hi ? hi : (uint32_t)pk;
    const bool ok = vbin(from_key(probe), bm) >= b;
    const uint64_t mask = __ballot(ok);  // lane 63 probes hi, so mask != 0
    const int f = __ffsll((unsigned long long)mask) - 1;
    const uint32_t nhi = (uint32_t)__builtin_amdgcn_readlane((int)probe, f);
    const uint32_t nlo = (f > 0) ? (uint32_t)__builtin_amdgcn_readlane((int)probe, f - 1) : lo;
    lo = nlo;
    hi = nhi;
  }
  return from_key(hi);
}


// Barrier over the G workgroups of one row (split tier).  Arrivals add one
// to the slot's counter, which only the row's last finishing workgroup
// returns to zero, so a workgroup's n-th barrier is passed once the counter
// reaches n * G (`nbar` counts this workgroup's barriers).  Everything that
// crosses between workgroups is an agent-scope atomic (adds, loads, stores),
// so no cache write-back or invalidate is needed: each wave only waits for
// its own atomics to complete before the workgroup arrives.  Spins are
// bounded (sy.spins polls): a wait that gives up adds one to the library's
// per-device timeout count (read by topk_status) and the workgroup moves on
// (that call's results are then undefined, but every wave exits).
__device__ __forceinline__ void row_barrier(SlotHeader* hdr, int G, uint32_t& nbar,
                                            const BarrierSync& sy) {
  wait_vm();
  __syncthreads();
  ++nbar;
  if (threadIdx.x == 0) {
    atomic_add_agent_nr(&hdr->bar_count, 1u);
    const uint32_t target = nbar * (uint32_t)G;
    uint32_t spins = 0;
    while (load_agent(&hdr->bar_count) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > sy.spins) {
        atomic_add_agent_nr(sy.err, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Count this workgroup as done with its row's slot; true in the last one.
// What the others wrote for it (list entries, counters) are agent-scope
// atomics they completed before counting themselves.
__device__ __forceinline__ bool finish_slot(SlotHeader* hdr, int G, uint32_t* bc) {
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) *bc = atomic_add_agent(&hdr->done, 1u);
  __syncthreads();
  return *bc == (uint32_t)(G - 1);
}

// Return a row's slot to its resting state (all zero): the histogram from bin
// hist_lo up (no round adds below its floor), the digit rows when `dig`, and
// the header.
__device__ __forceinline__ void rest_slot(SlotFixed* sf, int t, int block, int hist_lo, bool dig) {
  if (dig) {
    for (int i = t; i < 8 * 256; i += block) (&sf->dig[0][0])[i] = 0u;
    if (t < 16) sf->hdr.class_ext[t] = 0u;
  }
  for (int i = hist_lo + t; i < kBins; i += block) sf->hist[i] = 0u;
  if (t == 0) {
    sf->hdr.bar_count = 0u;
    sf->hdr.win_cur = 0u;
    sf->hdr.cand_cur = 0u;
    sf->hdr.tie_cur = 0u;
    sf->hdr.done = 0u;
  }
}

// ---------------------------------------------------------------------------
// Exact radix selection over an element set
// ---------------------------------------------------------------------------

struct RSel {
  uint32_t thr;    // key >> shift of the threshold digit path
  int shift;       // the lowest bit of the fixed digits (0 for a whole key)
  uint32_t rem;    // how many of the elements with key >> shift == thr to take
  uint32_t cnt;    // how many elements have key >> shift == thr
  int levels;      // digit levels counted
};

// The `need` largest keys among the elements `iter` visits (iter(f) calls
// f(key) for each element this thread owns): digit levels of DB bits from the
// top (the last level takes what is left of the 32 bits: 8-bit digits give
// four levels, 11-bit ones three of 11, 11 and 10 bits), stopping early when
// the crossing digit's members are all needed.  Afterwards an element is
// selected iff key >> shift > thr, or key >> shift == thr and it is one of
// `rem` such elements.  `dh` holds 2^DB LDS words.  With `gdig` (split
// rescue) the digit counts of the row's G workgroups are summed through the
// workspace (one row of 2^DB words per level) behind a barrier at each
// level.  Each level also finds the extremes of the class it counts (the
// keys that share the digits fixed so far), through `mm` (2 * BLOCK / 64 LDS
// words) and, split, the eight `gext` words (atomic max, zero at rest): a
// class holding a single key (all-equal rows, the ties of a two-valued row, a
// zero class) ends the selection with that key at once instead of after every
// level.  With EXT false (callers short of VGPRs) the extremes are not
// tracked.
template <int BLOCK, bool AGG = false, bool EXT = false, int DB = 8, class Iter>
__device__ __forceinline__ RSel radix_select(Iter&& iter, uint32_t need, uint32_t* dh, Cross* cross,
                                             uint32_t* scan, uint32_t* mm, uint32_t* gdig,
                                             uint32_t* gext, SlotHeader* hdr, int G,
                                             uint32_t& nbar, const BarrierSync& sy) {
  constexpr int W = BLOCK / 64;
  constexpr int NB = 1 << DB;
  constexpr int NL = (32 + DB - 1) / DB;
  static_assert(NL <= 4, "class extremes are kept for four levels");
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  uint32_t prefix = 0, rem = need, cnt = 0;
  int shift = 32, L = 0;
  while (L < NL) {
    const int hs = shift;  // the digits from bit hs up are fixed
    shift = 32 - DB * (L + 1) > 0 ? 32 - DB * (L + 1) : 0;
    const uint32_t dmask = (2u << (hs - shift - 1)) - 1u;
    for (int i = t; i < NB; i += BLOCK) dh[i] = 0u;
    lds_sync();
    uint32_t kmax = 0u, knmin = 0u;  // the class's largest key, smallest complemented
    iter([&](uint32_t key) {
      const bool act = L == 0 || ((key ^ prefix) >> hs) == 0u;
      const uint32_t d = (key >> shift) & dmask;
      if (AGG)
        lds_inc_agg(dh, d, act);
      else if (act)
        lds_inc(&dh[d]);
      if (EXT && act) {
        kmax = max(kmax, key);
        knmin = max(knmin, ~key);
      }
    });
    if (EXT) {
      wave_max2_u32(kmax, knmin);
      if (lane_id() == 0) {
        mm[w] = kmax;
        mm[W + w] = knmin;
      }
    }
    lds_sync();
    if (EXT) {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        kmax = max(kmax, (uint32_t)__builtin_amdgcn_readfirstlane((int)mm[i]));
        knmin = max(knmin, (uint32_t)__builtin_amdgcn_readfirstlane((int)mm[W + i]));
      }
    }
    if (gdig) {
      uint32_t* gd = gdig + L * NB;
      for (int i = t; i < NB; i += BLOCK) {
        const uint32_t c = dh[i];
        if (c) atomic_add_agent_nr(&gd[i], c);
      }
      if (EXT && t == 0) {
        if (kmax) __hip_atomic_fetch_max(&gext[L], kmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (knmin)
          __hip_atomic_fetch_max(&gext[4 + L], knmin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      row_barrier(hdr, G, nbar, sy);
      // the merged extremes are loaded first, so that their round trip is
      // the counts' own
      uint32_t gmx = 0u, gmn = 0u;
      if (EXT) {
        gmx = load_agent(&gext[L]);
        gmn = load_agent(&gext[4 + L]);
      }
      find_crossing<NB, BLOCK>([&](int d) { return load_agent(&gd[d]); }, rem, cross, scan);
      if (EXT) {
        kmax = (uint32_t)__builtin_amdgcn_readfirstlane((int)gmx);
        knmin = (uint32_t)__builtin_amdgcn_readfirstlane((int)gmn);
      }
    } else {
      find_crossing<NB, BLOCK>([&](int d) { return dh[d]; }, rem, cross, scan);
    }
    ++L;
    const Cross c = read_cross(cross);
    prefix |= (uint32_t)c.b << shift;
    rem -= c.above;
    cnt = c.m;
    if (c.m == rem) break;
    if (EXT && kmax == ~knmin) {
      // one key in the class: all of it sits in the crossing digit, and that
      // key is the threshold
      prefix = kmax;
      shift = 0;
      break;
    }
  }
  return RSel{prefix >> shift, shift, rem, cnt, L};
}

// The `need` largest of the m (key, index) pairs held in LDS, written from
// out[base] on (those in the K-th key's digit class after the others): an
// 8-bit radix select over the keys.  With `det`, when the K-th key's class
// holds more members than are needed, a second radix select over the
// complemented indices of that class (non-members count as key 0) keeps the
// smallest indices: that class then always ends with every member of its last
// digit needed, so the choice involves no ticket.  `ctr` is two LDS words,
// zero on entry.
template <int BLOCK>
__device__ __forceinline__ void list_select(const uint32_t* key, const int32_t* idx, uint32_t m,
                                            uint32_t need, bool det, int32_t* out, uint32_t base,
                                            uint32_t limit, uint32_t* dh, Cross* cross,
                                            uint32_t* scan, uint32_t* mm, uint32_t* ctr,
                                            uint32_t& nbar) {
  const int t = threadIdx.x;
  const RSel s = radix_select<BLOCK>(
      [&](auto&& f) {
        for (uint32_t i = t; i < m; i += BLOCK) f(key[i]);
      },
      need, dh, cross, scan, mm, nullptr, nullptr, nullptr, 1, nbar, BarrierSync{});
  const bool pick = det && s.cnt > s.rem;
  RSel s2{0u, 0, 0u, 0u};
  if (pick) {
    const uint32_t tk = s.thr;  // the select ended on one exact key
    s2 = radix_select<BLOCK>(
        [&](auto&& f) {
          for (uint32_t i = t; i < m; i += BLOCK) f(key[i] == tk ? ~(uint32_t)idx[i] : 0u);
        },
        s.rem, dh, cross, scan, mm, nullptr, nullptr, nullptr, 1, nbar, BarrierSync{});
  }
  const uint32_t eq_base = base + (need - s.rem);
  for (uint32_t i = t; i < m; i += BLOCK) {
    const uint32_t d = key[i] >> s.shift;
    if (d > s.thr) {
      const uint32_t pos = base + lds_take(&ctr[0]);
      if (pos < limit) out[pos] = idx[i];
    } else if (d == s.thr && (!pick || ((~(uint32_t)idx[i]) >> s2.shift) >= s2.thr)) {
      const uint32_t tk = lds_take(&ctr[1]);
      if (tk < s.rem && eq_base + tk < limit) out[eq_base + tk] = idx[i];
    }
  }
}

constexpr int kRankMax = 256;  // refine by rank counting up to this many candidates

}  // namespace ert

#endif  // ERT_GVR_DEVICE_H_
