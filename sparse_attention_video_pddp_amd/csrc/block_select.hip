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
// Kernels: pool_kernel (one workgroup per tile of Q or K: fp32 sums in a
// fixed order, then the mean; one read of Q and K) and block_select_kernel
// (one workgroup per query block: the block scores in LDS as order keys, the
// block select of select.hpp for the top J = min(nkb, ceil((k-1)/64) + 1)
// blocks, which always hold at least k tokens, then a rank walk over those J
// and the token emission).
#include "mcs_kernels.hpp"
#include "select.hpp"

namespace mcs {
namespace {

constexpr int kSelThreads = 256;

struct PoolParams {
  const void *Q, *K;
  float *qbar, *kbar;
  int Nq, Nkv, G, c, nkb, BH;
};

template <typename T, int D>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 x = *(const bf16x4*)p;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (float)x[e];
  } else {
    const f32x4 x = *(const f32x4*)p;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x[e];
  }
}

// Workgroups [0, BH*c) pool query tiles, the rest key tiles.  Thread
// (r, c4) sums channels 4*c4..4*c4+3 over rows r, r + RP, ...; the RP
// partial sums are then added in row-slot order.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  constexpr int C4 = D / 4, RP = 256 / C4;
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
  const int r = threadIdx.x / C4, c4 = threadIdx.x - r * C4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int row = r0 + r; row < r1; row += RP) {
    float v[4];
    load4<T, D>(src + (size_t)row * D + 4 * c4, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) part[r][4 * c4 + e] = acc[e];
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
  int Nq, Nkv, G, k, c, nkb, J;
  float scale;
  int causal_block, q_offset;
};

struct LdsKeys {
  const uint32_t* a;
  __device__ __forceinline__ uint32_t operator()(int j) const { return a[j]; }
};

template <int D>
__global__ __launch_bounds__(kSelThreads) void block_select_kernel(SelectParams p) {
  using Sel = BlockSelect<kSelThreads, 0>;
  __shared__ typename Sel::Shared sh;
  __shared__ uint32_t keys[kMaxKvBlocks];
  __shared__ __attribute__((aligned(16))) float qb[D];
  __shared__ int s_blk[kMaxSelBlocks], s_cnt[kMaxSelBlocks], s_off[kMaxSelBlocks], s_order[kMaxSelBlocks];
  __shared__ uint32_t s_key[kMaxSelBlocks];
  const int unit = blockIdx.x;
  const int bh = unit / p.c, g = unit - bh * p.c;
  const int tid = threadIdx.x;
  const int q0 = g * p.G, q1 = min(q0 + p.G, p.Nq);
  for (int i = tid; i < q1 - q0; i += kSelThreads) p.perm[(size_t)bh * p.Nq + q0 + i] = q0 + i;
  if (tid < D) qb[tid] = p.qbar[(size_t)unit * D + tid];
  __syncthreads();
  // the last query of the block sees the most keys (limits are nondecreasing)
  const int lim = visible_limit(q1 - 1, p.causal_block, p.q_offset, p.Nkv);
  for (int b = tid; b < p.nkb; b += kSelThreads) {
    const float* kr = p.kbar + ((size_t)bh * p.nkb + b) * D;
    float s = 0.f;
#pragma unroll 8
    for (int e = 0; e < D; e += 4) {
      const f32x4 kv = *(const f32x4*)(kr + e);
      const f32x4 qv = *(const f32x4*)(qb + e);
      s = fmaf(qv[0], kv[0], s);
      s = fmaf(qv[1], kv[1], s);
      s = fmaf(qv[2], kv[2], s);
      s = fmaf(qv[3], kv[3], s);
    }
    // order key of the score; blocks with no visible key take 0, below every score
    keys[b] = b * kPoolBlock < lim ? float_order_key(s * p.scale + 0.f) : 0u;
  }
  __syncthreads();
  const LdsKeys kf{keys};
  Sel sel;
  sel.n = p.nkb;
  uint32_t T;
  int tie_need;
  sel.threshold(kf, p.J, sh, T, tie_need);
  sel.split(kf, T, tie_need, sh, [&](int, int j, bool s, int pos) {
    if (s && pos < p.J) {
      s_blk[pos] = j;
      s_key[pos] = keys[j];
    }
  });
  __syncthreads();
  // score rank of each of the J blocks (they are in index order, so a lower
  // position is a lower block index)
  for (int e = tid; e < p.J; e += kSelThreads) {
    const uint32_t ke = s_key[e];
    int r = 0;
    for (int f = 0; f < p.J; ++f) r += (s_key[f] > ke) || (s_key[f] == ke && f < e);
    s_order[r] = e;
  }
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int r = 0; r < p.J; ++r) {
      const int e = s_order[r];
      const int size = min(kPoolBlock, p.Nkv - s_blk[e] * kPoolBlock);
      const int cnt = min(size, p.k - tot);
      s_cnt[e] = cnt;
      tot += cnt;
    }
    int off = 0;
    for (int e = 0; e < p.J; ++e) {
      s_off[e] = off;
      off += s_cnt[e];
    }
  }
  __syncthreads();
  int32_t* out = p.idx + (size_t)unit * p.k;
  const int t = tid & (kPoolBlock - 1);
  for (int e = tid / kPoolBlock; e < p.J; e += kSelThreads / kPoolBlock)
    if (t < s_cnt[e]) out[s_off[e] + t] = s_blk[e] * kPoolBlock + t;
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
  const dim3 sgrid((unsigned)((long long)s.BH * s.c));
  if (s.d == 128) hipLaunchKernelGGL(block_select_kernel<128>, sgrid, dim3(kSelThreads), 0, st, sp);
  else hipLaunchKernelGGL(block_select_kernel<64>, sgrid, dim3(kSelThreads), 0, st, sp);
  return hipGetLastError();
}

}  // namespace mcs
