// Shared machinery of the flash-style kernels: the direct-to-LDS K/V tile
// ring and the per-wave online-softmax core over one or more 32-key blocks.
//
// LDS tile layout.  A tile holds TK rows of K followed by TK rows of V, d
// channels each, unpadded.  Rows arrive by global_load_lds_dwordx4 (lane i of
// a wave-wide load writes 16 bytes at base + 16*i), so every row is stored as
// its 16-byte chunks with chunk c placed at chunk c ^ swz(r).  The swizzle
// keeps the 16-byte K-operand reads (one chunk of 8 or 16 consecutive rows)
// and the transposing V reads (4 consecutive rows x 2 chunks) free of bank
// conflicts; it depends on r only through r mod 16, so every 32-row block of a
// tile has the same internal layout.
//
// Per-wave core.  One wave owns 32 query columns.  Scores are formed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so a lane owns one
// query column and 16 keys of the block: softmax max/sum are in-lane plus one
// exchange of the wave halves, and the probabilities already sit in the B
// operand layout of O^T = V^T P^T, whose V^T operand is read with
// ds_read_b64_tr_b16.  Softmax runs in base 2 with scale*log2(e) folded into
// one FMA; the reference maximum is only moved when a block exceeds it by
// more than 2^8 (lazy rescaling; exact after the final division by the sum).
#pragma once

#include "mcs_device.hpp"

namespace mcs {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kRescaleSlack = 8.0f;  // log2 units

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte chunk c of row r sits at chunk c ^ swz(r) of the LDS row.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 2 * (r & 7) + ((r >> 3) & 1);
  else return 2 * (r & 3) + ((r >> 2) & 1);
}

// Direct-to-LDS copy of one 16-byte chunk per lane (wave-uniform LDS base).
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_base, 16, 0, 0);
}

// Buffer resource over [base, base + bytes) for raw (stride 0) buffer loads:
// a lane whose offset falls outside reads zeros.  bytes < 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Direct-to-LDS copy of 16 bytes per lane at byte offset voff of a buffer
// (wave-uniform LDS base, lane i writes base + 16*i).
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, voff, 0, 0, 0);
}

template <int D>
struct FlashCore {
  static constexpr int NB = D / 32;   // 32-channel output blocks
  static constexpr int NKS = D / 16;  // k-steps of QK^T
  bf16x8 qb[NKS];
  f32x16 acc[NB];
  float m_run, l_run;
  // Per-lane LDS byte offsets in XOR form (see block32).
  int kbase, vbase0, vbase1;

  __device__ __forceinline__ void init(const __bf16* qrow, bool valid) {
    const int l = lane_id(), n = l & 31, h = l >> 5;
    kbase = n * (2 * D) + 16 * (h ^ swz<D>(n));
    const int vr = 4 * h + ((l & 15) >> 2);
    const int c0 = 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
    vbase0 = vr * (2 * D) + 8 * (l & 1) + 16 * (c0 ^ swz<D>(vr));
    vbase1 = (8 + vr) * (2 * D) + 8 * (l & 1) + 16 * (c0 ^ swz<D>(8 + vr));
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 z = {};
      qb[ks] = valid ? *(const bf16x8*)(qrow + ks * 16 + 8 * h) : z;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
    m_run = -kInf;
    l_run = 0.f;
  }

  // Scores S^T of NKB consecutive 32-key blocks (K rows at Ks, blocks BLK
  // bytes apart).  Element i of block kb holds key 32*kb + 8*(i/4) + 4*h + i%4.
  // The K operand of k-step ks (row n, chunk (2ks+h) ^ swz(n)) is
  // Ks + (kbase ^ 32*ks): one XOR per read, constant offsets.
  template <int NKB, int BLK>
  __device__ __forceinline__ void scores(const unsigned char* Ks, f32x16 (&s)[NKB]) const {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a = *(const bf16x8*)(Ks + kb * BLK + (kbase ^ (32 * ks)));
        s[kb] = mfma_32x32x16(a, qb[ks], s[kb]);
      }
    }
  }

  // Online softmax of the scores s (one update for all NKB blocks) and the
  // O^T += V^T P^T product (V rows at Vs, blocks BLK bytes apart).  lim: keys
  // of these blocks visible to this lane's query (any integer).  The V^T
  // operand of channel block b (rows 16*ks2 + 8*hi + vr, chunk (4b + c0) ^
  // swz(row)) is Vs + (vbase_hi ^ 64*b) + 16*ks2 rows.
  template <int NKB, int BLK>
  __device__ __forceinline__ void softmax_pv(f32x16 (&s)[NKB], const unsigned char* Vs, int lim, float c) {
    const int h = lane_id() >> 5;
    // element i of block kb holds key 32*kb + 8*(i/4) + 4*h + i%4; mask keys >= lim
    const int lh = lim - 4 * h;
    if (lh < 32 * NKB - 4) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb + 8 * (i >> 2) + (i & 3) >= lh) s[kb][i] = -kInf;
    }
    float mx = -kInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = half_max(mx) * c;
    const float m_new = (mx > m_run + kRescaleSlack) ? mx : m_run;
    const float m_ref = (m_new == -kInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] *= alpha;
    }
    // per 32-key block: probabilities, then O^T += V^T P^T.  A operand slot j
    // of lane (d = l%32, half h) is key 16*ks2 + 8*(j/4) + 4*h + j%4 (the key
    // of slot j of this lane's P^T)
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      bf16x8 pb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(fmaf(s[kb][i], c, -m_ref));
        ls += pv;
        pb[i >> 3][i & 7] = (__bf16)pv;
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int a0 = vbase0 ^ (64 * b), a1 = vbase1 ^ (64 * b);
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          const bf16x4 lo = lds_read_tr(Vs + kb * BLK + a0 + 16 * (2 * D) * ks2);
          const bf16x4 hi = lds_read_tr(Vs + kb * BLK + a1 + 16 * (2 * D) * ks2);
          acc[b] = mfma_32x32x16(cat(lo, hi), pb[ks2], acc[b]);
        }
      }
    }
    l_run = fmaf(l_run, alpha, ls);
  }

  // One pipelined step: softmax and O^T += V^T P^T of the tile whose scores
  // are in s (V rows at Vs, lim visible keys), with the scores of the next
  // tile (K rows at Kn) formed into sn in between.  The two rare branches
  // (masking, rescaling O) come first, so the next tile's MFMAs, this tile's
  // exponentials and its PV MFMAs share one basic block and can be
  // interleaved.  Kn may be any tile of LDS when there is no next tile (sn is
  // then unused).
  template <int NKB, int BLK>
  __device__ __forceinline__ void step(f32x16 (&s)[NKB], const unsigned char* Vs, int lim, float c,
                                       const unsigned char* Kn, f32x16 (&sn)[NKB]) {
    const int h = lane_id() >> 5;
    const int lh = lim - 4 * h;
    if (lh < 32 * NKB - 4) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb + 8 * (i >> 2) + (i & 3) >= lh) s[kb][i] = -kInf;
    }
    float mx = -kInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = half_max(mx) * c;
    const float m_new = (mx > m_run + kRescaleSlack) ? mx : m_run;
    const float m_ref = (m_new == -kInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] *= alpha;
    }
    scores<NKB, BLK>(Kn, sn);
    float ls = 0.f;
    bf16x8 pb[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(fmaf(s[kb][i], c, -m_ref));
        ls += pv;
        pb[kb][i >> 3][i & 7] = (__bf16)pv;
      }
    l_run = fmaf(l_run, alpha, ls);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int a0 = vbase0 ^ (64 * b), a1 = vbase1 ^ (64 * b);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          const bf16x4 lo = lds_read_tr(Vs + kb * BLK + a0 + 16 * (2 * D) * ks2);
          const bf16x4 hi = lds_read_tr(Vs + kb * BLK + a1 + 16 * (2 * D) * ks2);
          acc[b] = mfma_32x32x16(cat(lo, hi), pb[kb][ks2], acc[b]);
        }
    }
  }

  // Both steps on one tile.
  template <int NKB, int BLK>
  __device__ __forceinline__ void blocks(const unsigned char* Ks, const unsigned char* Vs, int lim, float c) {
    f32x16 s[NKB];
    scores<NKB, BLK>(Ks, s);
    softmax_pv<NKB, BLK>(s, Vs, lim, c);
  }

  // 1 / row sum (0 for a row with no visible key) and the natural-log lse.
  __device__ __forceinline__ float finish(float& lse) const {
    const float lt = half_sum(l_run);
    lse = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -kInf;
    return lt > 0.f ? 1.f / lt : 0.f;
  }

  // Output element (b, i) of a lane is channel b*32 + 8*(i/4) + 4*h + i%4.
  __device__ __forceinline__ f32x4 out4(int b, int q4, float inv) const {
    return f32x4{acc[b][4 * q4] * inv, acc[b][4 * q4 + 1] * inv, acc[b][4 * q4 + 2] * inv,
                 acc[b][4 * q4 + 3] * inv};
  }
};

}  // namespace mcs
