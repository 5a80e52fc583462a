// Block-sparse comparator: mean-pooled block selection, recomputed every step.
//
// MC-Sparse review (blog.secrett2633.cloud), section 1 (selection error of
// approximate scoring such as mean pooling; structural binding error of
// whole-block selection) and section 2 (block-sparse attention imposes
// sparsity at block granularity, which suits GPU tiles).  This is the
// selection MC-Sparse's reused exact token selection is compared with.
//
// Query blocks are the G-token tiles of the token order (so the grouping is
// the identity) and KV blocks the 64-token tiles, the K/V tile of the
// attention kernels; each last tile may be short.  A block is represented by
// the mean of its rows; the score of KV block b for query block g is
// scale * <mean q_g, mean k_b>.  KV blocks with no key visible to any query of
// g rank after all others.  Blocks are taken by decreasing score (ties to the
// lower block index) while the token count stays within k; the next block
// then gives its lowest-index tokens up to exactly k.  The token lists are
// written ascending and feed the gathered sparse attention unchanged.
//
// Kernels.  pool_kernel: one workgroup per tile of Q or K, fp32 sums in a
// fixed order, then the mean (one read of Q and K).  The select kernels run
// one workgroup per query block.  Scores: eight lanes per pooled key row
// (coalesced 512-byte rows, all loads of a pass in flight), summed in a fixed
// butterfly.  Ranking: with at most kSortBlocks KV blocks, a bitonic sort in
// LDS of (score key, block index) pairs; beyond, the radix block select of
// select.hpp for the top J = min(nkb, ceil((k-1)/64) + 1) blocks (which always
// hold at least k tokens) followed by an exact ranking of those J.  The token
// counts of the ranked blocks come from one scan of their sizes, their output
// offsets from one scan in block-index order.
#include "mcs_kernels.hpp"
#include "select.hpp"

namespace mcs {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSortBlocks = 4096;  // bitonic path limit (32 KB of pairs)

struct PoolParams {
  const void *Q, *K;
  float *qbar, *kbar;
  int Nq, Nkv, G, c, nkb, BH;
};

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
  } else {
    const f32x4 x0 = *(const f32x4*)p, x1 = *(const f32x4*)(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = x0[e];
      v[4 + e] = x1[e];
    }
  }
}

// Workgroups [0, BH*c) pool query tiles, the rest key tiles.  Thread
// (r, c8) sums channels 8*c8..8*c8+7 over rows r, r + RP, ... (16-byte loads
// of bf16, all of a thread's rows in flight); the RP partial sums are then
// added in row-slot order.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  constexpr int C8 = D / 8, RP = 256 / C8, MAXR = 128 / RP;  // tiles have at most 128 rows
  __shared__ float part[RP][D];
  int unit = blockIdx.x;
  const T* src;
  float* dst;
  int r0, r1;
  if (unit < p.BH * p.c) {
    const int bh = unit / p.c, t = unit - bh * p.c;
    r0 = t * p.G;
    r1 = min(r0 + p.G, p.Nq);
    src = (const T*)p.Q + (size_t)bh * p.Nq * D;
    dst = p.qbar + (size_t)unit * D;
  } else {
    unit -= p.BH * p.c;
    const int bh = unit / p.nkb, t = unit - bh * p.nkb;
    r0 = t * kPoolBlock;
    r1 = min(r0 + kPoolBlock, p.Nkv);
    src = (const T*)p.K + (size_t)bh * p.Nkv * D;
    dst = p.kbar + (size_t)unit * D;
  }
  const int r = threadIdx.x / C8, c8 = threadIdx.x - r * C8;
  float v[MAXR][8];
#pragma unroll
  for (int i = 0; i < MAXR; ++i)
    if (i * RP < r1 - r0) {  // uniform; within it, rows past the tile are clamped, loaded and not added
      const int row = min(r0 + r + i * RP, r1 - 1);
      load8<T>(src + (size_t)row * D + 8 * c8, v[i]);
    }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MAXR; ++i)
    if (r0 + r + i * RP < r1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[i][e];
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r][8 * c8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) s += part[i][threadIdx.x];
    dst[threadIdx.x] = s / (float)(r1 - r0);
  }
}

struct SelectParams {
  const float *qbar, *kbar;
  int32_t *perm, *idx;
  int Nq, Nkv, G, k, c, nkb, J, npad;
  float scale;
  int causal_block, q_offset;
};

struct LdsKeys {
  const uint32_t* a;
  __device__ __forceinline__ uint32_t operator()(int j) const { return a[j]; }
};

// Identity grouping of this query block and its pooled vector into LDS.
template <int D>
__device__ __forceinline__ void select_prologue(const SelectParams& p, int unit, float* qb) {
  const int bh = unit / p.c, g = unit - bh * p.c;
  const int q0 = g * p.G, q1 = min(q0 + p.G, p.Nq);
  for (int i = threadIdx.x; i < q1 - q0; i += kSelThreads) p.perm[(size_t)bh * p.Nq + q0 + i] = q0 + i;
  if (threadIdx.x < D) qb[threadIdx.x] = p.qbar[(size_t)unit * D + threadIdx.x];
  __syncthreads();
}

// Order key of every KV block's score (0 for a block with no visible key,
// below every score); put(b, key) for b < nkb.  Eight lanes share a row: lane
// `sub` multiplies channels [sub*D/8, (sub+1)*D/8) in order, then the eight
// partial sums meet in a fixed butterfly.
template <int D, class Put>
__device__ __forceinline__ void block_scores(const SelectParams& p, int unit, const float* qb, Put&& put) {
  constexpr int LPR = 8, CPL = D / LPR, RPP = kSelThreads / LPR, U = 4;
  const int bh = unit / p.c, g = unit - bh * p.c;
  const int q1 = min(g * p.G + p.G, p.Nq);
  // the last query of the block sees the most keys (limits are nondecreasing)
  const int lim = visible_limit(q1 - 1, p.causal_block, p.q_offset, p.Nkv);
  const int sub = threadIdx.x & (LPR - 1), rr = threadIdx.x / LPR;
  float qv[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) qv[i] = qb[sub * CPL + i];
  const float* kh = p.kbar + (size_t)bh * p.nkb * D + sub * CPL;
  for (int b0 = 0; b0 < p.nkb; b0 += RPP * U) {
    float part[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = min(b0 + u * RPP + rr, p.nkb - 1);
      const f32x4* kr = (const f32x4*)(kh + (size_t)b * D);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < CPL / 4; ++i) {
        const f32x4 v = kr[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) sum = fmaf(qv[4 * i + e], v[e], sum);
      }
      part[u] = sum;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sum = part[u];
      sum += __shfl_xor(sum, 1, 64);
      sum += __shfl_xor(sum, 2, 64);
      sum += __shfl_xor(sum, 4, 64);
      const int b = b0 + u * RPP + rr;
      if (sub == 0 && b < p.nkb) put(b, b * kPoolBlock < lim ? float_order_key(sum * p.scale + 0.f) : 0u);
    }
  }
}

// Token counts of the J ranked blocks (rank r: block blk[r], kPoolBlock
// tokens but the last block's), taken in rank order up to k in all:
// cnt[r].  sw: scan scratch.  Ends with a barrier.
__device__ __forceinline__ void rank_counts(const SelectParams& p, const int* blk, int* cnt, int* sw) {
  const int tid = threadIdx.x;
  int sz[2], tot;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 2 * tid + h;
    sz[h] = r < p.J ? min(kPoolBlock, p.Nkv - blk[r] * kPoolBlock) : 0;
  }
  int run = block_excl_scan<kSelThreads>(sz[0] + sz[1], sw, tot);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 2 * tid + h;
    if (r < p.J) cnt[r] = max(0, min(sz[h], p.k - run));
    run += sz[h];
  }
  __syncthreads();
}

// Exclusive scan of n <= PER * kSelThreads ints (PER contiguous per thread)
// into out.  Ends with a barrier.
template <int PER, class In>
__device__ __forceinline__ void scan_blocked(int n, In&& in, int* out, int* sw) {
  int loc[PER], s = 0, tot;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int b = PER * threadIdx.x + i;
    loc[i] = b < n ? in(b) : 0;
    s += loc[i];
  }
  int off = block_excl_scan<kSelThreads>(s, sw, tot);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int b = PER * threadIdx.x + i;
    if (b < n) out[b] = off;
    off += loc[i];
  }
  __syncthreads();
}

// Tokens of J chosen blocks: entry i is block blocks[i], cnts[i] tokens
// written from offs[i].  One wave per entry, lane t its t-th token.
__device__ __forceinline__ void emit_tokens(const SelectParams& p, int unit, const int* blocks, const int* cnts,
                                            const int* offs) {
  int32_t* out = p.idx + (size_t)unit * p.k;
  const int t = threadIdx.x & 63;
  for (int i = threadIdx.x >> 6; i < p.J; i += kSelThreads / 64)
    if (t < cnts[i]) out[offs[i] + t] = blocks[i] * kPoolBlock + t;
}

// Descending bitonic sort of n (a power of two) 64-bit values in LDS.
__device__ __forceinline__ void bitonic_sort_desc(unsigned long long* a, int n) {
  for (int size = 2; size <= n; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int q = threadIdx.x; q < n / 2; q += kSelThreads) {
        const int i = 2 * stride * (q / stride) + (q % stride), j = i + stride;
        const bool desc = (i & size) == 0;  // the final merge (size == n) is descending throughout
        const unsigned long long x = a[i], y = a[j];
        if ((x < y) == desc) {
          a[i] = y;
          a[j] = x;
        }
      }
      __syncthreads();
    }
}

// Up to kSortBlocks KV blocks.  Dynamic LDS: npad 64-bit (key, ~block)
// pairs, reused after the sort for per-block counts and offsets [nkb] each;
// then three arrays of J: ranked blocks, their counts and output offsets.
template <int D>
__global__ __launch_bounds__(kSelThreads) void block_select_sort_kernel(SelectParams p) {
  __shared__ __attribute__((aligned(16))) float qb[D];
  __shared__ int sw[kSelThreads / 64];
  extern __shared__ unsigned long long dyn64[];
  unsigned long long* comp = dyn64;
  int* blk = (int*)(dyn64 + p.npad);
  int* cnt = blk + p.J;
  int* offr = cnt + p.J;
  const int unit = blockIdx.x;
  select_prologue<D>(p, unit, qb);
  // higher key first, then lower block index; padding (0) sorts last
  for (int b = p.nkb + threadIdx.x; b < p.npad; b += kSelThreads) comp[b] = 0ull;
  block_scores<D>(p, unit, qb, [&](int b, uint32_t key) {
    comp[b] = ((unsigned long long)key << 32) | (0xFFFFFFFFu - (uint32_t)b);
  });
  __syncthreads();
  bitonic_sort_desc(comp, p.npad);
  for (int r = threadIdx.x; r < p.J; r += kSelThreads) blk[r] = (int)(0xFFFFFFFFu - (uint32_t)comp[r]);
  __syncthreads();
  rank_counts(p, blk, cnt, sw);
  // output offsets in block-index order: counts scattered by block, one scan
  int* cntb = (int*)comp;
  int* offb = cntb + p.nkb;
  for (int b = threadIdx.x; b < p.nkb; b += kSelThreads) cntb[b] = 0;
  __syncthreads();
  for (int r = threadIdx.x; r < p.J; r += kSelThreads) cntb[blk[r]] = cnt[r];
  __syncthreads();
  scan_blocked<kSortBlocks / kSelThreads>(p.nkb, [&](int b) { return cntb[b]; }, offb, sw);
  for (int r = threadIdx.x; r < p.J; r += kSelThreads) offr[r] = offb[blk[r]];
  __syncthreads();
  emit_tokens(p, unit, blk, cnt, offr);
}

// More than kSortBlocks KV blocks (up to kMaxKvBlocks).  Dynamic LDS: keys
// [nkb], then six arrays of J: the selected blocks in index order, their
// keys, their ranks, the blocks in rank order, the counts by rank, and
// counts then offsets in index order.
template <int D>
__global__ __launch_bounds__(kSelThreads) void block_select_radix_kernel(SelectParams p) {
  using Sel = BlockSelect<kSelThreads, 0>;
  __shared__ typename Sel::Shared sh;
  __shared__ __attribute__((aligned(16))) float qb[D];
  extern __shared__ uint32_t dyn[];
  uint32_t* keys = dyn;
  int* s_sel = (int*)(keys + p.nkb);
  uint32_t* s_key = (uint32_t*)(s_sel + p.J);
  int* rk = (int*)(s_key + p.J);
  int* blk = rk + p.J;
  int* cnt = blk + p.J;
  int* cnte = cnt + p.J;
  int* offe = (int*)s_key;  // the keys are no longer needed once the counts are known
  const int unit = blockIdx.x;
  select_prologue<D>(p, unit, qb);
  block_scores<D>(p, unit, qb, [&](int b, uint32_t key) { keys[b] = key; });
  __syncthreads();
  const LdsKeys kf{keys};
  Sel sel;
  sel.n = p.nkb;
  uint32_t T;
  int tie_need;
  sel.threshold(kf, p.J, sh, T, tie_need);
  sel.split(kf, T, tie_need, sh, [&](int, int j, bool s, int pos) {
    if (s && pos < p.J) {
      s_sel[pos] = j;
      s_key[pos] = keys[j];
    }
  });
  __syncthreads();
  // rank of each selected block by (key desc, index asc); they are in index
  // order, so a lower position is a lower block index
  for (int e = threadIdx.x; e < p.J; e += kSelThreads) {
    const uint32_t ke = s_key[e];
    int r = 0;
    for (int f = 0; f < p.J; ++f) r += (s_key[f] > ke) || (s_key[f] == ke && f < e);
    rk[e] = r;
    blk[r] = s_sel[e];
  }
  __syncthreads();
  rank_counts(p, blk, cnt, sh.cnt_eq);
  for (int e = threadIdx.x; e < p.J; e += kSelThreads) cnte[e] = cnt[rk[e]];
  __syncthreads();
  scan_blocked<kMaxSelBlocks / kSelThreads>(p.J, [&](int e) { return cnte[e]; }, offe, sh.cnt_eq);
  emit_tokens(p, unit, s_sel, cnte, offe);
}

}  // namespace

size_t block_workspace_bytes(const Shape& s) {
  const size_t nkb = (size_t)(s.Nkv + kPoolBlock - 1) / kPoolBlock;
  return (size_t)s.BH * ((size_t)s.c + nkb) * s.d * 4;
}

hipError_t launch_block_select(const Shape& s, bool bf16, const void* Q, const void* K, int32_t* perm,
                               int32_t* idx, void* ws, hipStream_t st) {
  const int nkb = (s.Nkv + kPoolBlock - 1) / kPoolBlock;
  float* qbar = (float*)ws;
  float* kbar = qbar + (size_t)s.BH * s.c * s.d;
  const PoolParams pp{Q, K, qbar, kbar, s.Nq, s.Nkv, s.G, s.c, nkb, s.BH};
  const dim3 pgrid((unsigned)((long long)s.BH * (s.c + nkb)));
  if (bf16 && s.d == 128) hipLaunchKernelGGL((pool_kernel<__bf16, 128>), pgrid, dim3(256), 0, st, pp);
  else if (bf16) hipLaunchKernelGGL((pool_kernel<__bf16, 64>), pgrid, dim3(256), 0, st, pp);
  else if (s.d == 128) hipLaunchKernelGGL((pool_kernel<float, 128>), pgrid, dim3(256), 0, st, pp);
  else hipLaunchKernelGGL((pool_kernel<float, 64>), pgrid, dim3(256), 0, st, pp);
  SelectParams sp;
  sp.qbar = qbar; sp.kbar = kbar; sp.perm = perm; sp.idx = idx;
  sp.Nq = s.Nq; sp.Nkv = s.Nkv; sp.G = s.G; sp.k = s.k; sp.c = s.c; sp.nkb = nkb;
  sp.J = block_select_count(s.k, nkb);
  sp.scale = s.scale; sp.causal_block = s.causal_block; sp.q_offset = s.q_offset;
  int npad = 64;
  while (npad < nkb) npad *= 2;
  sp.npad = npad;
  const dim3 sgrid((unsigned)((long long)s.BH * s.c));
  if (nkb <= kSortBlocks) {
    const size_t lds = (size_t)npad * 8 + (size_t)sp.J * 12;  // <= 38 KB
    if (s.d == 128) hipLaunchKernelGGL(block_select_sort_kernel<128>, sgrid, dim3(kSelThreads), lds, st, sp);
    else hipLaunchKernelGGL(block_select_sort_kernel<64>, sgrid, dim3(kSelThreads), lds, st, sp);
  } else {
    const size_t lds = ((size_t)nkb + (size_t)sp.J * 6) * 4;  // <= 44 KB (+ 18 KB static)
    if (s.d == 128) hipLaunchKernelGGL(block_select_radix_kernel<128>, sgrid, dim3(kSelThreads), lds, st, sp);
    else hipLaunchKernelGGL(block_select_radix_kernel<64>, sgrid, dim3(kSelThreads), lds, st, sp);
  }
  return hipGetLastError();
}

}  // namespace mcs
