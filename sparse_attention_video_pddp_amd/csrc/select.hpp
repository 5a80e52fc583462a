// Exact block-wide selection of the `need` largest 32-bit keys of an array,
// equal keys taken lowest index first, followed by an order-preserving split
// of the array into the selected and the remaining elements.
//
// Used for the per-group token-level top-k (MC-Sparse review,
// blog.secrett2633.cloud, section 3: each query group keeps the KV tokens of
// largest exact attention mass) and for the rank split of every PDDP node
// (the floor(c/2)*G members of smallest projection go left; the caller flips
// the projection keys so that "smallest" becomes "largest").
//
// Element j of the array belongs to thread j % NT ("stripe" j / NT).  With
// VPT > 0 the caller caches the keys of its VPT stripes in registers (the
// array must then hold at most VPT * NT elements); with VPT == 0 keys are
// re-read through a functor on every pass (four reads in all), sixteen
// stripes' keys loaded before any is used (one load in flight per thread
// left these reads latency-bound: 14.5 -> 6 ms for the top-k of 16384 rows
// of 131072 masses).  Positions j >= n of the last
// stripe read as key 0: they sit above every real index, so they are never
// selected ahead of a real key (at most n are selected) and every stripe can
// be processed without lane masks; only the final emit skips them.
//
// Threshold: three MSB-first radix passes (12, 12 and 8 bits, or 12, 12 and
// HI-24 bits for keys below 2^HI) over the elements whose key matches the
// digits found so far; histograms in LDS.
// The result is the need-th largest key T and how many keys equal to T are
// selected.
//
// Split: per (stripe, wave) the counts of keys > T and == T come from two
// ballots; one block scan over these counts gives every wave its offsets, so
// each element knows its rank among the selected (or the remaining) elements
// in index order without further synchronisation.  Stripes are handled in
// blocks of 64 (three barriers per block).
#pragma once

#include "mcs_device.hpp"

namespace mcs {

// Inclusive prefix sum over one 64-lane wave by DPP moves: shifts within each
// row of 16 lanes (the first three from the original values, then by 4 and 8
// in the upper banks), then the last lane of row 0 into row 1 and of row 2
// into row 3, then lane 31 into rows 2 and 3.  No LDS permutes.
__device__ __forceinline__ int wave_incl_scan_dpp(int x) {
  int s = x + __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  s += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);          // row_shr:2
  s += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xF, 0xF, true);          // row_shr:3
  s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xF, 0xE, true);          // row_shr:4, lanes 4..15 of a row
  s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xF, 0xC, true);          // row_shr:8, lanes 8..15
  s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xA, 0xF, false);         // row_bcast:15 into rows 1, 3
  s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xC, 0xF, false);         // row_bcast:31 into rows 2, 3
  return s;
}

// Exclusive block scan over NT threads; `total` receives the block sum.
// Two barriers; s_w holds NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* s_w, int& total) {
  constexpr int NW = NT / 64;
  const int w = wave_id();
  const int x = wave_incl_scan_dpp(v);
  if (lane_id() == 63) s_w[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int s = s_w[i];
    off += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return x - v + off;
}

template <int NT, int VPT>
struct BlockSelect {
  static_assert(NT % 64 == 0 && NT >= 256 && NT <= 1024, "block size");
  static constexpr int NW = NT / 64;
  static constexpr int NBIN = 4096;
  static constexpr int BPT = NBIN / NT;  // histogram bins owned by one thread in the rank search
  static constexpr int VB = 64;         // stripes per split block (one per lane; VB * NW <= NT)
  static_assert(VPT >= 0, "register cache");

  // LDS layouts padded against bank conflicts: histogram bin b at
  // b + b / BPT (the BPT bins a thread scans are consecutive, so lanes land
  // BPT + 1 words apart, an odd stride); split entry e = (stripe slot l,
  // wave w) = l * NW + w at e + e / NW (written by lane l of wave w: stride
  // NW + 1).
  static __device__ __forceinline__ int hidx(int b) { return b + b / BPT; }
  static __device__ __forceinline__ int eidx(int e) { return e + e / NW; }

  struct Shared {
    int hist[NBIN + NBIN / BPT];
    int cnt_gt[VB * (NW + 1)];
    int cnt_eq[VB * (NW + 1)];
    int wsum[NW];
    uint32_t prefix;
    int krem;
  };

  uint32_t v[VPT > 0 ? VPT : 1];  // cached keys of stripes 0..VPT-1 (VPT > 0)
  int n;                          // array length

  // Key of position j in register mode: a clamped (unconditional) read.
  template <class Keys>
  __device__ __forceinline__ void load(const Keys& keys) {
    if constexpr (VPT > 0) {
      // an opaque copy of the thread index keeps the compiler from holding
      // these positions (and their range tests) live until the split
      int t = threadIdx.x;
      asm volatile("" : "+v"(t));
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int j = i * NT + t;
        const uint32_t u = keys(min(j, n - 1));
        v[i] = j < n ? u : 0u;
      }
    }
  }

  // f(stripe, j, key) for the stripes [s0, s1) of this thread (uniform trip
  // count).  In register mode s0 and s1 are compile-time after unrolling
  // (whole blocks of VB stripes, also those past the end, keys 0 — see
  // above), so no per-stripe conditions stay live.
  template <class Keys, class F>
  __device__ __forceinline__ void stripes(int s0, int s1, const Keys& keys, F&& f) const {
    const int t = threadIdx.x;
    if constexpr (VPT > 0) {
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (i >= s0 && i < s1) f(i, i * NT + t, v[i]);
    } else {
      constexpr int U = 16;
      int s = s0;
      for (; s + U <= s1; s += U) {
        uint32_t u[U];
#pragma unroll
        for (int i = 0; i < U; ++i) u[i] = keys(min((s + i) * NT + t, n - 1));
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const int j = (s + i) * NT + t;
          f(s + i, j, j < n ? u[i] : 0u);
        }
      }
      for (; s < s1; ++s) {
        const int j = s * NT + t;
        const uint32_t u = keys(min(j, n - 1));
        f(s, j, j < n ? u : 0u);
      }
    }
  }

  // T = need-th largest key (1 <= need <= n); tie_need = how many keys equal
  // to T belong to the selection.  HI: keys are below 2^HI (31 for the bit
  // patterns of non-negative floats), so the first pass takes bits
  // [HI-12, HI) and the last the HI-24 lowest bits.
  template <int HI = 32, class Keys>
  __device__ void threshold(const Keys& keys, int need, Shared& sh, uint32_t& T, int& tie_need) const {
    static_assert(HI >= 25 && HI <= 32, "three passes of at most 12 bits");
    const int t = threadIdx.x;
    const int top = NBIN - 1 - t * BPT;  // this thread's bins: top, top-1, ..., top-BPT+1
#pragma unroll
    for (int b = 0; b < BPT; ++b) sh.hist[hidx(top - b)] = 0;
    __syncthreads();
    const int nstripes = VPT > 0 ? VPT : (n + NT - 1) / NT;
    uint32_t prefix = 0, pmask = 0;
    int krem = need;  // rank, from the top, still to locate among keys matching prefix
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? HI - 12 : (pass == 1 ? HI - 24 : 0);
      const uint32_t dmask = pass == 2 ? (1u << (HI - 24)) - 1u : 0xFFFu;
      stripes(0, nstripes, keys, [&](int, int, uint32_t u) {
        const bool m = (u & pmask) == prefix;
        if (__ballot(m)) {  // later passes: most stripes hold no matching key
          if (m) atomicAdd(&sh.hist[hidx((u >> shift) & dmask)], 1);
        }
      });
      __syncthreads();
      int cnt[BPT], local = 0;
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        cnt[b] = sh.hist[hidx(top - b)];
        local += cnt[b];
      }
      int total;
      const int above = block_excl_scan<NT>(local, sh.wsum, total);  // matching keys in higher bins
      if (above < krem && above + local >= krem) {
        int c = above;
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
          if (c + cnt[b] >= krem) {
            sh.prefix = prefix | ((uint32_t)(top - b) << shift);
            sh.krem = krem - c;
            break;
          }
          c += cnt[b];
        }
      }
#pragma unroll
      for (int b = 0; b < BPT; ++b) sh.hist[hidx(top - b)] = 0;
      __syncthreads();
      prefix = sh.prefix;
      krem = sh.krem;
      pmask |= dmask << shift;
    }
    T = prefix;
    tie_need = krem;
  }

  // Set bits of a wave mask held by lanes below this one.
  static __device__ __forceinline__ int below_count(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  }

  // emit(stripe, j, selected, pos) for every element j < n: pos is the rank
  // of j among the selected elements, or among the remaining ones, in index
  // order.
  template <class Keys, class Emit>
  __device__ void split(const Keys& keys, uint32_t T, int tie_need, Shared& sh, Emit&& emit) const {
    const int w = wave_id(), l = lane_id();
    const int nstripes = VPT > 0 ? VPT : (n + NT - 1) / NT;
    int base_eq = 0, base_sel = 0;
    auto block = [&](int s0, int s1) {
      // lane i of each wave collects the counts of stripe s0 + i (VB == 64 lanes)
      int my_gt = 0, my_eq = 0;
      stripes(s0, s1, keys, [&](int s, int, uint32_t u) {
        const int gtc = __popcll(__ballot(u > T)), eqc = __popcll(__ballot(u == T));
        my_gt = (l == s - s0) ? gtc : my_gt;
        my_eq = (l == s - s0) ? eqc : my_eq;
      });
      if (l < s1 - s0) {
        sh.cnt_gt[eidx(l * NW + w)] = my_gt;
        sh.cnt_eq[eidx(l * NW + w)] = my_eq;
      }
      __syncthreads();
      const int e = threadIdx.x;  // entry (stripe s0 + e / NW, wave e % NW), in index order
      const bool ein = e < (s1 - s0) * NW;
      const int eqc = ein ? sh.cnt_eq[eidx(e)] : 0, gtc = ein ? sh.cnt_gt[eidx(e)] : 0;
      int eq_tot, sel_tot;
      const int eq_off = base_eq + block_excl_scan<NT>(eqc, sh.wsum, eq_tot);
      const int selc = gtc + min(max(tie_need - eq_off, 0), eqc);
      const int sel_off = base_sel + block_excl_scan<NT>(selc, sh.wsum, sel_tot);
      if (ein) {
        sh.cnt_eq[eidx(e)] = eq_off;
        sh.cnt_gt[eidx(e)] = sel_off;
      }
      __syncthreads();
      const int my_eo = l < s1 - s0 ? sh.cnt_eq[eidx(l * NW + w)] : 0;
      const int my_so = l < s1 - s0 ? sh.cnt_gt[eidx(l * NW + w)] : 0;
      stripes(s0, s1, keys, [&](int s, int j, uint32_t u) {
        bool sel = u > T;
        const uint64_t eqm = __ballot(u == T);
        if (eqm) {  // rare: keys equal to T, taken lowest index first
          const int eo = __builtin_amdgcn_readlane(my_eo, s - s0);  // ties before this stripe's wave slice
          sel = sel || (u == T && eo + below_count(eqm) < tie_need);
        }
        const int so = __builtin_amdgcn_readlane(my_so, s - s0);  // selections before it
        const int before = so + below_count(__ballot(sel));       // selected elements with a lower index
        if (j < n) emit(s, j, sel, sel ? before : j - before);
      });
      base_eq += eq_tot;
      base_sel += sel_tot;
      if (s1 < nstripes) __syncthreads();  // the counts are reused by the next block
    };
    if constexpr (VPT > 0) {
#pragma unroll
      for (int s0 = 0; s0 < VPT; s0 += VB) block(s0, s0 + VB < VPT ? s0 + VB : VPT);
    } else {
      for (int s0 = 0; s0 < nstripes; s0 += VB) block(s0, min(nstripes, s0 + VB));
    }
  }
};

}  // namespace mcs
