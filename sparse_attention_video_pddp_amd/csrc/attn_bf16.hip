// bf16 attention kernels on gfx950 MFMA: exact dense attention and the
// anchor's per-group column mass.
//
// Method: MC-Sparse review (blog.secrett2633.cloud), section "3. Method & Key
// Results": exact scores at the anchor step, from which each query group's
// token-level KV selection is made.  (The gathered sparse attention of the
// reuse step is in sparse_bf16.hip.)
//
// Shared structure.  One wave owns 32 query rows.  K/V tiles of 64 keys are
// staged in LDS (row-major; K rows padded so 16-lane 16-byte reads hit
// distinct banks, V rows padded for the transposing reads) with a register
// prefetch of the next tile.  Scores are formed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16, so each lane holds 32 keys of one query column:
// the softmax max/sum are in-lane plus one exchange of the two wave halves,
// and the probabilities already sit in the B-operand layout of the
// O^T = V^T P^T product (the A operand V^T comes from ds_read_b64_tr_b16).
// Online softmax runs in base 2 with scale*log2(e) folded into one FMA.
#include <type_traits>

#include "mcs_kernels.hpp"
#include "ring.hpp"

namespace mcs {
namespace {

template <int D>
struct Tile {
  static constexpr int KS = D + 8;   // K row stride (elements)
  static constexpr int VS = D + 32;  // V row stride (elements)
  static constexpr int CH = D / 8;   // 16-byte chunks per row
};

// Register staging of one 64-key tile: global -> registers -> LDS.  Loads are
// buffer loads over the tile's rows: the per-thread byte offsets never change
// (no address arithmetic per tile) and rows past the end of the head read as
// zeros (their keys are masked).
template <int D, int NT>
struct TileStage {
  static constexpr int CH = D / 8;
  static constexpr int N = 64 * CH / NT;
  static_assert(N >= 1 && (64 * CH) % NT == 0, "tile/thread mismatch");
  u32x4 kr[N];
  u32x4 vr[N];

  __device__ __forceinline__ void load(const __bf16* K, const __bf16* V, int row0, int nrows) {
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(K + (size_t)row0 * D, nrows * D * 2);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(V + (size_t)row0 * D, nrows * D * 2);
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ci = t + i * NT;
      const int off = (ci / CH) * (2 * D) + (ci % CH) * 16;
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  }
  __device__ __forceinline__ void store(__bf16* Ks, __bf16* Vs) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ci = t + i * NT;
      const int r = ci / CH, col = (ci % CH) * 8;
      *(u32x4*)(Ks + r * Tile<D>::KS + col) = kr[i];
      *(u32x4*)(Vs + r * Tile<D>::VS + col) = vr[i];
    }
  }
};

// Flash-attention state of one wave (32 query columns).
template <int D>
struct Flash {
  static constexpr int NB = D / 32;
  static constexpr int NKS = D / 16;
  bf16x8 qb[NKS];
  f32x16 acc[NB];
  float m_run, l_run;

  __device__ __forceinline__ void init(const __bf16* qrow, bool valid) {
    const int h = lane_id() >> 5;
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

  // One 64-key tile.  lim: how many leading keys of the tile are visible to
  // this lane's query (any integer; >= 64 means all).  c = scale*log2(e).
  // MASK = false: every key of the tile is visible to every query of the
  // wave (no masking code, so nothing divergent separates the QK MFMAs from
  // the maximum).
  template <bool MASK>
  __device__ __forceinline__ void tile(const __bf16* Ks, const __bf16* Vs, int lim, float c) {
    const int l = lane_id(), n = l & 31, h = l >> 5;
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a = *(const bf16x8*)(Ks + (kb * 32 + n) * Tile<D>::KS + ks * 16 + 8 * h);
        s[kb] = mfma_32x32x16(a, qb[ks], s[kb]);
      }
    }
    if (MASK && lim < 64) {
      const int lh = lim - 4 * h;  // element i of block kb is key kb*32 + 8*(i/4) + 4*h + i%4
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i >> 2) + (i & 3) >= lh) s[kb][i] = -kInf;
    }
    float mx = -kInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = half_max(mx) * c;
    // Lazy rescaling: keep the reference maximum unless this tile exceeds it
    // by more than 2^8 (probabilities stay <= 256, far from fp32/bf16 limits;
    // the final normalisation by the row sum makes the result exact).
    const float m_new = (mx > m_run + kRescaleSlack) ? mx : m_run;
    const float m_ref = (m_new == -kInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    m_run = m_new;
    float ls4[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short dependency chains
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[kb][i], c, -m_ref));
        ls4[i & 3] += p;
        pb[kb][i >> 3][i & 7] = (__bf16)p;
      }
    l_run = fmaf(l_run, alpha, (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]));
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] *= alpha;
    }
    // O^T += V^T P^T.  A operand lane (d = l%32, half h), slot j holds key
    // kb*32 + 16*ks2 + 8*(j/4) + 4*h + j%4, the key whose probability sits in
    // slot j of this lane's B operand.
    const int vrow = 4 * h + ((l & 15) >> 2);
    const int vcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          const __bf16* vp = Vs + (kb * 32 + 16 * ks2 + vrow) * Tile<D>::VS + b * 32 + vcol;
          acc[b] = mfma_32x32x16(cat(lds_read_tr(vp), lds_read_tr(vp + 8 * Tile<D>::VS)), pb[kb][ks2],
                                 acc[b]);
        }
    // the row-sum update stays in this block, beside the PV MFMAs (left to
    // itself the compiler sinks it past the next tile's LDS stores, where it
    // issues alone)
    asm volatile("" : "+v"(l_run));
  }

  // 1 / row sum (0 for a row with no visible key) and the natural-log lse.
  __device__ __forceinline__ float finish(float& lse) {
    const float lt = half_sum(l_run);
    lse = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -kInf;
    return lt > 0.f ? 1.f / lt : 0.f;
  }
};

// Output element (b, i) of a lane is d = b*32 + 8*(i/4) + 4*h + i%4: four
// consecutive channels per (b, i/4).
template <int D>
__device__ __forceinline__ void store_row_bf16(__bf16* dst, const Flash<D>& st, float inv, const float* add) {
  const int h = lane_id() >> 5;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = b * 32 + 8 * g + 4 * h;
      f32x4 v = {st.acc[b][4 * g] * inv, st.acc[b][4 * g + 1] * inv, st.acc[b][4 * g + 2] * inv,
                 st.acc[b][4 * g + 3] * inv};
      if (add) v += *(const f32x4*)(add + d0);
      bf16x4 o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
      *(bf16x4*)(dst + d0) = o;
    }
}

template <int D>
__device__ __forceinline__ void store_row_f32(float* dst, const Flash<D>& st, float inv, bool subtract) {
  const int h = lane_id() >> 5;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = b * 32 + 8 * g + 4 * h;
      f32x4 v = {st.acc[b][4 * g] * inv, st.acc[b][4 * g + 1] * inv, st.acc[b][4 * g + 2] * inv,
                 st.acc[b][4 * g + 3] * inv};
      if (subtract) v = *(const f32x4*)(dst + d0) - v;
      *(f32x4*)(dst + d0) = v;
    }
}

// ---------------------------------------------------------------------------
// Dense attention, natural token order: 256 queries (8 waves) per workgroup,
// so one staged K/V tile serves eight waves (against four: 6.80 -> 6.39 ms at
// 32760 tokens, 12 heads, d = 128; 84.3 -> 80.1 ms at 131072 tokens, 16
// heads, d = 64).  Two waves per SIMD at d = 128 (230 registers), four at
// d = 64 (123).  Two LDS tiles, one barrier per tile.
// ---------------------------------------------------------------------------
struct DenseParams {
  const __bf16 *Q, *K, *V;
  __bf16* O;
  float* lse;
  float* Ofull;
  int Nq, Nkv, n_qtiles, n_units, per_xcd;
  float c;
  int causal_block, q_offset;
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 2, D == 64 ? 4 : 2))) void dense_bf16_kernel(DenseParams p) {
  constexpr int NT = 64 * NW, QR = 32 * NW;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][64 * Tile<D>::KS];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][64 * Tile<D>::VS];
  const int unit = xcd_unit(blockIdx.x, p.per_xcd);
  if (unit >= p.n_units) return;
  const int bh = unit / p.n_qtiles, qt = unit - bh * p.n_qtiles;
  const int w = wave_id(), n = lane_id() & 31, h = lane_id() >> 5;
  const int q = qt * QR + w * 32 + n;
  const bool qv = q < p.Nq;
  const int vcount = qv ? visible_limit(q, p.causal_block, p.q_offset, p.Nkv) : 0;
  const int kmax = visible_limit(min(qt * QR + QR, p.Nq) - 1, p.causal_block, p.q_offset, p.Nkv);
  const int ntiles = (kmax + 63) / 64;
  const __bf16* Kh = p.K + (size_t)bh * p.Nkv * D;
  const __bf16* Vh = p.V + (size_t)bh * p.Nkv * D;
  Flash<D> st;
  st.init(p.Q + ((size_t)bh * p.Nq + (qv ? q : 0)) * D, qv);
  TileStage<D, NT> stage;
  stage.load(Kh, Vh, 0, p.Nkv);
  stage.store(Ks[0], Vs[0]);
  __syncthreads();
  // two LDS tiles: tile t + 1 is stored into the other buffer while tile t is
  // used; one barrier per tile (the buffer written was last read before the
  // previous barrier)
  auto step = [&](int t, auto maskc) {
    const int base = t * 64, cur = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) stage.load(Kh, Vh, base + 64, p.Nkv - base - 64);
    st.template tile<decltype(maskc)::value>(Ks[cur], Vs[cur], vcount - base, p.c);
    if (more) stage.store(Ks[cur ^ 1], Vs[cur ^ 1]);
    __syncthreads();
  };
  // the first nfull tiles are visible in full to every query of the
  // workgroup (its first query sees the fewest keys) and need no masking:
  // 6.25 -> 6.00 ms at 32760 tokens, 12 heads; 1.12 -> 0.92 ms for a
  // frame-causal chunk of 4680 queries over 32760 keys
  const int nfull = min(ntiles, visible_limit(min(qt * QR, p.Nq - 1), p.causal_block, p.q_offset, p.Nkv) / 64);
  int t = 0;
  for (; t < nfull; ++t) step(t, std::false_type{});
  for (; t < ntiles; ++t) step(t, std::true_type{});
  float lse;
  const float inv = st.finish(lse);
  if (qv) {
    const size_t row = (size_t)bh * p.Nq + q;
    store_row_bf16<D>(p.O + row * D, st, inv, nullptr);
    if (p.Ofull) store_row_f32<D>(p.Ofull + row * D, st, inv, false);
    if (p.lse && h == 0) p.lse[row] = lse;
  }
}

// ---------------------------------------------------------------------------
// Anchor column mass: m_g[j] = sum_{i in g} exp(scale*<q_i,k_j> - lse_i).
// Scores are formed as S = Q K^T here so that a lane holds one key column.
// Each wave owns 64 queries as two 32-row MFMA blocks that share every K
// operand read from LDS (half the LDS traffic per MFMA of a 32-query wave);
// a lane's mass over the wave's 64 queries is in-lane plus one half-wave
// exchange.  A 64-query group is one wave and its sums go straight to
// memory; a 128-query group is two waves whose sums meet in LDS.
// ---------------------------------------------------------------------------
struct MassParams {
  const __bf16 *Q, *K;
  const int32_t* perm;
  const float* lse;
  float* mass;
  int Nq, Nkv, c, bh0, upb, n_units, per_xcd;
  float c_log2;
  int causal_block, q_offset;
  int nsplit, tps;  // key ranges per query block, 64-key tiles per range
};

template <int D, int NW>
struct MassTile {
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int RPL = 64 / CH;        // rows per wave-wide copy
  static constexpr int LPW = 64 / RPL / NW;  // copies per wave per 64-key tile
  static constexpr int BYTES = 64 * D * 2;
};

// NW waves (64 * NW queries) per workgroup over one range of tps K tiles
// (the mass of a key depends on no other key, so workloads with few query
// blocks split the keys to fill the chip).  K tiles of 64 keys arrive by
// direct-to-LDS copies in a two-slot ring (row layout and swizzle of
// ring.hpp), one barrier per tile; for two-wave groups that barrier also
// orders the per-wave sums of the previous tile (double-buffered) before they
// are added.  Per-query lse and visibility limits are staged in LDS: the lse
// values are read once into registers, the limits only by tiles that some
// query of the wave sees in part.  Three waves per SIMD at d = 128 (within
// 168 registers), four at d = 64: the exponentials and the per-score VALU
// work of one wave run beside the MFMAs of the others.
template <int D, int G, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 3, D == 64 ? 4 : 3))) void mass_bf16_kernel(MassParams p) {
  using T = MassTile<D, NW>;
  constexpr int QR = 64 * NW, WPG = G / 64, GPW = QR / G, NKS = D / 16;
  static_assert(WPG == 1 || WPG == 2, "group size");
  static_assert(T::LPW >= 1, "copies per wave");
  __shared__ __attribute__((aligned(1024))) unsigned char k0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[T::BYTES];
  __shared__ float part[WPG > 1 ? 2 : 1][NW][64];
  __shared__ __attribute__((aligned(16))) float s_lse[NW][64];
  __shared__ __attribute__((aligned(16))) int s_lim[NW][64];
  __shared__ int s_kmax[NW];
  const int unit = xcd_unit(blockIdx.x, p.per_xcd);
  if (unit >= p.n_units) return;
  const int qunit = unit / p.nsplit, ksp = unit - qunit * p.nsplit;
  const int bhl = qunit / p.upb, u = qunit - bhl * p.upb;
  const int bh = p.bh0 + bhl;
  const int w = wave_id(), l = lane_id(), n = l & 31, h = l >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int pos0 = u * QR + w * 64;
  const int32_t* hperm = p.perm + (size_t)bh * p.Nq;
  // query pos0 + l: its row, lse (base 2; padding rows +inf so they add 0) and limit
  int lmax, lmin;
  {
    const bool v = pos0 + l < p.Nq;
    const int row = v ? min(max(hperm[pos0 + l], 0), p.Nq - 1) : 0;
    const float ls = p.lse[(size_t)bh * p.Nq + row];
    s_lse[w][l] = (!v || ls == -kInf) ? kInf : ls * kLog2e;
    const int lim = v ? visible_limit(row, p.causal_block, p.q_offset, p.Nkv) : 0;
    s_lim[w][l] = lim;
    lmax = lim;
    lmin = v ? lim : p.Nkv;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lmax = max(lmax, __shfl_xor(lmax, o, 64));
    lmin = min(lmin, __shfl_xor(lmin, o, 64));
  }
  bf16x8 qa[2][NKS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const bool v = pos0 + 32 * qb + n < p.Nq;
    const int row = v ? min(max(hperm[pos0 + 32 * qb + n], 0), p.Nq - 1) : 0;
    const __bf16* qp = p.Q + ((size_t)bh * p.Nq + row) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 z = {};
      qa[qb][ks] = v ? *(const bf16x8*)(qp + ks * 16) : z;
    }
  }
  if (l == 0) s_kmax[w] = lmax;
  __syncthreads();
  int kmax = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) kmax = max(kmax, s_kmax[i]);
  const int t0 = ksp * p.tps;
  const int ntiles = max(0, min((kmax + 63) / 64, t0 + p.tps) - t0);  // tiles t0 .. t0 + ntiles - 1
  // score row i of block qb on this lane: query 32*qb + 8*(i/4) + 4*h + i%4 of the wave
  float lse2[2][16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 v4 = *(const f32x4*)&s_lse[w][32 * qb + 8 * r + 4 * h];
#pragma unroll
      for (int e = 0; e < 4; ++e) lse2[qb][4 * r + e] = v4[e];
    }
  const __bf16* Kh = p.K + (size_t)bh * p.Nkv * D;
  const int kbase = n * (2 * D) + 16 * (h ^ swz<D>(n));
  int voff[T::LPW];
#pragma unroll
  for (int j = 0; j < T::LPW; ++j) {
    const int r = T::RPL * (wu + NW * j) + l / T::CH;
    voff[j] = r * (2 * D) + (((l % T::CH) ^ swz<D>(r)) * 16);
  }
  // rows past the end of the head read as zeros (their keys are masked)
  auto issue = [&](int i, unsigned char* slot) {
    const int t = t0 + i;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(Kh + (size_t)t * 64 * D, (p.Nkv - t * 64) * D * 2);
#pragma unroll
    for (int j = 0; j < T::LPW; ++j) dma16_buf(r, voff[j], slot + (wu + NW * j) * 1024);
  };
  // group sums of tile t0 + i, whose per-wave sums are in part[b] (two-wave groups)
  auto reduce = [&](int i, int b) {
    if constexpr (WPG > 1) {
      const int t = t0 + i;
      if (threadIdx.x < GPW * 64) {
        const int gl = threadIdx.x >> 6, key = threadIdx.x & 63;
        const float m = part[b][2 * gl][key] + part[b][2 * gl + 1][key];
        const int gg = u * GPW + gl;
        if (gg < p.c && t * 64 + key < p.Nkv) p.mass[((size_t)bhl * p.c + gg) * p.Nkv + t * 64 + key] = m;
      }
    }
  };
  auto tile = [&](int i, const unsigned char* Ks, int b) {
    const int base = (t0 + i) * 64;
    const bool full = base + 64 <= lmin;  // every key of the tile visible to every query of the wave
    float cs2[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s[2] = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 kk = *(const bf16x8*)(Ks + kb * 32 * 2 * D + (kbase ^ (32 * ks)));
        s[0] = mfma_32x32x16(qa[0][ks], kk, s[0]);
        s[1] = mfma_32x32x16(qa[1][ks], kk, s[1]);
      }
      float cs = 0.f;
      if (full) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 16; ++i) cs += fast_exp2(fmaf(s[qb][i], p.c_log2, -lse2[qb][i]));
      } else {
        const int key = base + kb * 32 + n;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int4 lm = *(const int4*)&s_lim[w][32 * qb + 8 * r + 4 * h];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pv = fast_exp2(fmaf(s[qb][4 * r + e], p.c_log2, -lse2[qb][4 * r + e]));
              cs += (key < lm[e]) ? pv : 0.f;
            }
          }
      }
      cs2[kb] = half_sum(cs);
    }
    // lane (h, n) holds key 32*h + n of the tile
    const float out = h ? cs2[1] : cs2[0];
    if constexpr (WPG == 1) {
      const int gg = u * GPW + w, key = base + 32 * h + n;
      if (gg < p.c && key < p.Nkv) p.mass[((size_t)bhl * p.c + gg) * p.Nkv + key] = out;
    } else {
      part[b][w][l] = out;
    }
  };
  if (ntiles > 0) {
    issue(0, k0);
    if (ntiles > 1) issue(1, k1);
  }
  for (int t = 0; t < ntiles; t += 2) {
    // K(t) landed; K(t+1), issued after it, may still be in flight
    if (t + 1 < ntiles) wait_vmcnt<T::LPW>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (t > 0) reduce(t - 1, 1);
    tile(t, k0, 0);
    if (t + 1 >= ntiles) break;
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 2 < ntiles) issue(t + 2, k0);
    reduce(t, 0);
    tile(t + 1, k1, 1);
    __syncthreads();
    if (t + 3 < ntiles) issue(t + 3, k1);
  }
  if constexpr (WPG > 1) {
    __syncthreads();
    if (ntiles > 0) reduce(ntiles - 1, (ntiles - 1) & 1);
  }
  // keys of this range past the last visible tile: no query of the
  // workgroup sees them, so their mass is 0 (every key of a row is written)
  const int z0 = (t0 + ntiles) * 64, z1 = min((t0 + p.tps) * 64, p.Nkv);
  for (int gl = 0; gl < GPW; ++gl) {
    const int gg = u * GPW + gl;
    if (gg >= p.c) break;
    float* row = p.mass + ((size_t)bhl * p.c + gg) * p.Nkv;
    for (int key = z0 + (int)threadIdx.x; key < z1; key += 64 * NW) row[key] = 0.f;
  }
}

template <typename P>
inline void grid_for(P& p, int units, dim3& grid) {
  p.n_units = units;
  p.per_xcd = (units + 7) / 8;
  grid = dim3(8 * p.per_xcd);
}

}  // namespace

hipError_t launch_dense_bf16(const Shape& s, const void* Q, const void* K, const void* V, void* O,
                             float* lse, float* Ofull, hipStream_t st) {
  DenseParams p;
  p.Q = (const __bf16*)Q; p.K = (const __bf16*)K; p.V = (const __bf16*)V; p.O = (__bf16*)O;
  p.lse = lse; p.Ofull = Ofull;
  const int qr = 256;  // 8 waves x 32 queries
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.n_qtiles = (s.Nq + qr - 1) / qr;
  p.c = s.scale * kLog2e; p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  dim3 grid;
  grid_for(p, s.BH * p.n_qtiles, grid);
  if (s.d == 128) hipLaunchKernelGGL((dense_bf16_kernel<128, 8>), grid, dim3(512), 0, st, p);
  else hipLaunchKernelGGL((dense_bf16_kernel<64, 8>), grid, dim3(512), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_mass_bf16(const Shape& s, int bh0, int nbh, const void* Q, const void* K,
                            const int32_t* perm, const float* lse, float* mass, hipStream_t st) {
  MassParams p;
  p.Q = (const __bf16*)Q; p.K = (const __bf16*)K; p.perm = perm; p.lse = lse; p.mass = mass;
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.c = s.c; p.bh0 = bh0;
  p.c_log2 = s.scale * kLog2e; p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  // four-wave workgroups (one K tile serves 256 queries); the keys are split
  // into ranges when the query blocks alone give fewer than ~6 waves per SIMD
  constexpr int kQR = 256, kWaveTarget = 6144;
  p.upb = (s.Nq + kQR - 1) / kQR;
  const int kt = (s.Nkv + 63) / 64;
  const long long waves = (long long)nbh * p.upb * (kQR / 64);
  int ns = (int)std::min<long long>((kWaveTarget + waves - 1) / waves, std::max(1, kt / 4));
  p.tps = (kt + ns - 1) / ns;
  p.nsplit = (kt + p.tps - 1) / p.tps;
  dim3 grid;
  grid_for(p, nbh * p.upb * p.nsplit, grid);
#define MCS_MASS(DD, GG) hipLaunchKernelGGL((mass_bf16_kernel<DD, GG, 4>), grid, dim3(256), 0, st, p)
  if (s.d == 128 && s.G == 64) MCS_MASS(128, 64);
  else if (s.d == 128) MCS_MASS(128, 128);
  else if (s.G == 64) MCS_MASS(64, 64);
  else MCS_MASS(64, 128);
#undef MCS_MASS
  return hipGetLastError();
}

}  // namespace mcs
