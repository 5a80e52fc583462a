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
    if (lim < 64) {
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

__device__ __forceinline__ int visible_limit(int qpos, int causal_block, int q_offset, int Nkv) {
  if (!causal_block) return Nkv;
  const long long lim = ((long long)(q_offset + qpos) / causal_block + 1) * causal_block;
  return lim < Nkv ? (int)lim : Nkv;
}

// ---------------------------------------------------------------------------
// Dense attention: 128 queries (4 waves) per workgroup, natural token order.
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

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void dense_bf16_kernel(DenseParams p) {
  constexpr int NT = 256, QR = 128;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[64 * Tile<D>::KS];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[64 * Tile<D>::VS];
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
  stage.store(Ks, Vs);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int base = t * 64;
    const bool more = t + 1 < ntiles;
    if (more) stage.load(Kh, Vh, base + 64, p.Nkv - base - 64);
    st.tile(Ks, Vs, vcount - base, p.c);
    __syncthreads();
    if (more) {
      stage.store(Ks, Vs);
      __syncthreads();
    }
  }
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
// 128 queries (4 waves) per workgroup = 128/G groups.  Scores are formed as
// S = Q K^T here so that a lane holds one key column: its mass over the
// wave's 32 queries is in-lane plus one half-wave exchange.
// ---------------------------------------------------------------------------
struct MassParams {
  const __bf16 *Q, *K;
  const int32_t* perm;
  const float* lse;
  float* mass;
  int Nq, Nkv, c, bh0, upb, n_units, per_xcd;
  float c_log2;
  int causal_block, q_offset;
};

template <int D>
struct MassTile {
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int RPL = 64 / CH;       // rows per wave-wide copy
  static constexpr int LPW = 64 / RPL / 4;  // copies per wave per 64-key tile
  static constexpr int BYTES = 64 * D * 2;
};

// K tiles of 64 keys arrive by direct-to-LDS copies in a two-slot ring (row
// layout and swizzle of ring.hpp); one barrier per tile, which also orders the
// per-wave column sums of the previous tile (double-buffered) before their
// reduction over the group's waves.  A tile that every query of the wave sees
// in full takes the unmasked path.  Three waves per SIMD: within 168
// registers the scores stay in VGPRs (no accumulator-register copies, which
// would cost VALU issue slots).
template <int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void mass_bf16_kernel(MassParams p) {
  using T = MassTile<D>;
  constexpr int QR = 128, GPW = QR / G, WPG = G / 32, NKS = D / 16;
  __shared__ __attribute__((aligned(1024))) unsigned char k0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[T::BYTES];
  __shared__ float part[2][4][64];
  __shared__ int s_kmax[4];
  const int unit = xcd_unit(blockIdx.x, p.per_xcd);
  if (unit >= p.n_units) return;
  const int bhl = unit / p.upb, u = unit - bhl * p.upb;
  const int bh = p.bh0 + bhl;
  const int w = wave_id(), l = lane_id(), n = l & 31, h = l >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int pos0 = u * QR + w * 32;
  const int32_t* hperm = p.perm + (size_t)bh * p.Nq;
  const float* hlse = p.lse + (size_t)bh * p.Nq;
  bf16x8 qa[NKS];
  {
    const bool v = pos0 + n < p.Nq;
    const int row = v ? min(max(hperm[pos0 + n], 0), p.Nq - 1) : 0;
    const __bf16* qp = p.Q + ((size_t)bh * p.Nq + row) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 z = {};
      qa[ks] = v ? *(const bf16x8*)(qp + ks * 16) : z;
    }
  }
  // per score row i of this lane: query 8*(i/4) + 4*h + i%4 of the wave
  float lse2[16];
  int lim[16];
  int lmax = 0, lmin = p.Nkv;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int qp = pos0 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (qp < p.Nq) {
      const int row = min(max(hperm[qp], 0), p.Nq - 1);
      const float ls = hlse[row];
      lse2[i] = (ls == -kInf) ? kInf : ls * kLog2e;
      lim[i] = visible_limit(row, p.causal_block, p.q_offset, p.Nkv);
      lmin = min(lmin, lim[i]);
    } else {
      lse2[i] = kInf;  // exp2(-inf) = 0: padding rows add nothing
      lim[i] = 0;
    }
    lmax = max(lmax, lim[i]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lmax = max(lmax, __shfl_xor(lmax, o, 64));
    lmin = min(lmin, __shfl_xor(lmin, o, 64));
  }
  if (l == 0) s_kmax[w] = lmax;
  __syncthreads();
  const int kmax = max(max(s_kmax[0], s_kmax[1]), max(s_kmax[2], s_kmax[3]));
  const int ntiles = (kmax + 63) / 64;
  const __bf16* Kh = p.K + (size_t)bh * p.Nkv * D;
  const int kbase = n * (2 * D) + 16 * (h ^ swz<D>(n));
  int voff[T::LPW];
#pragma unroll
  for (int j = 0; j < T::LPW; ++j) {
    const int r = T::RPL * (wu + 4 * j) + l / T::CH;
    voff[j] = r * (2 * D) + (((l % T::CH) ^ swz<D>(r)) * 16);
  }
  // rows past the end of the head read as zeros (their keys are masked)
  auto issue = [&](int t, unsigned char* slot) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(Kh + (size_t)t * 64 * D, (p.Nkv - t * 64) * D * 2);
#pragma unroll
    for (int j = 0; j < T::LPW; ++j) dma16_buf(r, voff[j], slot + (wu + 4 * j) * 1024);
  };
  // group sums of the tile whose per-wave sums are in part[b]
  auto reduce = [&](int t, int b) {
    if (threadIdx.x < GPW * 64) {
      const int gl = threadIdx.x >> 6, key = threadIdx.x & 63;
      float m = 0.f;
#pragma unroll
      for (int ww = 0; ww < WPG; ++ww) m += part[b][gl * WPG + ww][key];
      const int gg = u * GPW + gl;
      if (gg < p.c && t * 64 + key < p.Nkv) p.mass[((size_t)bhl * p.c + gg) * p.Nkv + t * 64 + key] = m;
    }
  };
  auto tile = [&](int t, const unsigned char* Ks, int b) {
    const int base = t * 64;
    const bool full = base + 64 <= lmin;  // every key of the tile visible to every query of the wave
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 kk = *(const bf16x8*)(Ks + kb * 32 * 2 * D + (kbase ^ (32 * ks)));
        s = mfma_32x32x16(qa[ks], kk, s);
      }
      float cs = 0.f;
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) cs += fast_exp2(fmaf(s[i], p.c_log2, -lse2[i]));
      } else {
        const int key = base + kb * 32 + n;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = fast_exp2(fmaf(s[i], p.c_log2, -lse2[i]));
          cs += (key < lim[i]) ? pv : 0.f;
        }
      }
      cs = half_sum(cs);
      if (h == 0) part[b][w][kb * 32 + n] = cs;
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
  __syncthreads();
  if (ntiles > 0) reduce(ntiles - 1, (ntiles - 1) & 1);
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
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.n_qtiles = (s.Nq + 127) / 128;
  p.c = s.scale * kLog2e; p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  dim3 grid;
  grid_for(p, s.BH * p.n_qtiles, grid);
  if (s.d == 128) hipLaunchKernelGGL(dense_bf16_kernel<128>, grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(dense_bf16_kernel<64>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_mass_bf16(const Shape& s, int bh0, int nbh, const void* Q, const void* K,
                            const int32_t* perm, const float* lse, float* mass, hipStream_t st) {
  MassParams p;
  p.Q = (const __bf16*)Q; p.K = (const __bf16*)K; p.perm = perm; p.lse = lse; p.mass = mass;
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.c = s.c; p.bh0 = bh0;
  const int gpw = 128 / s.G;
  p.upb = (s.c + gpw - 1) / gpw;
  p.c_log2 = s.scale * kLog2e; p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  dim3 grid;
  grid_for(p, nbh * p.upb, grid);
  if (s.d == 128 && s.G == 64) hipLaunchKernelGGL((mass_bf16_kernel<128, 64>), grid, dim3(256), 0, st, p);
  else if (s.d == 128) hipLaunchKernelGGL((mass_bf16_kernel<128, 128>), grid, dim3(256), 0, st, p);
  else if (s.G == 64) hipLaunchKernelGGL((mass_bf16_kernel<64, 64>), grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((mass_bf16_kernel<64, 128>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mcs
