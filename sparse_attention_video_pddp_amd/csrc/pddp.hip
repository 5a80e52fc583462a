// Fast-PDDP query grouping (MC-Sparse review, blog.secrett2633.cloud,
// section 3: similar queries are packed into equal-size, tile-aligned groups
// by Principal Direction Divisive Partitioning).
//
// The tree is processed level by level; at each level one workgroup owns one
// node, i.e. one contiguous range perm[start, start+n) of a head (groups are
// numbered depth-first, so every node stays contiguous).  For a node holding
// c >= 2 groups the workgroup
//   1. forms S = sum x and the raw scatter sum x x^T over the node's query
//      rows: bf16 rows through v_mfma_f32_32x32x16_bf16 (exact products,
//      fp32 accumulation over 64-row chunks, fp64 across chunks), fp32 rows
//      with fp64 FMA;
//   2. centres it, C = sum x x^T - S S^T / n (fp64), and runs the fixed-step
//      power iteration v <- C v / ||C v|| from v0 = 1/sqrt(d) in fp64
//      (a zero product keeps v);
//   3. projects p_i = (x_i - mean) . v in fp64 and stores an order key of
//      float(p_i);
//   4. radix-selects the (floor(c/2)*G)-th smallest key and stably partitions
//      the members (key, then position = original index, since members are
//      kept ascending) into the left and right child ranges.
// Wave w of the workgroup holds column block w of C in the MFMA output layout
// (lane: one column, 16 rows per 32-row block), so C v needs only an in-lane
// sum and one half-wave exchange (C is symmetric).
#include "mcs_device.hpp"
#include "mcs_kernels.hpp"

namespace mcs {
namespace {

struct PddpParams {
  const void* Q;
  int32_t* perm;
  int32_t* tmp;
  uint32_t* keys;
  int Nq, G, iters, level;
};

__device__ __forceinline__ int scan256(int v, int* s_wsum) {
  const int w = wave_id();
  const int x = wave_incl_scan(v);
  if (lane_id() == 63) s_wsum[w] = x;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) off += (i < w) ? s_wsum[i] : 0;
  __syncthreads();
  return x + off;
}

__global__ void pddp_init_kernel(int32_t* perm, int Nq, size_t total) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < total) perm[i] = (int32_t)(i % (size_t)Nq);
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void pddp_level_kernel(PddpParams p) {
  constexpr int NB = D / 32;
  constexpr int XS = 64 + 8;  // transposed bf16 staging: row = one channel, 64 query rows
  constexpr int FS = D + 4;   // fp32 staging: row = one query row
  constexpr int STAGE_BYTES = BF16 ? D * XS * 2 : 64 * FS * 4;
  __shared__ __attribute__((aligned(16))) unsigned char stage_raw[STAGE_BYTES];
  __shared__ double sS[D], sV[D];
  __shared__ double sRed[4];
  __shared__ int hist[256];
  __shared__ int s_wsum[4];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;
  __shared__ int s_tot[2];

  const int bh = blockIdx.y, slot = blockIdx.x;
  int start = 0, n = p.Nq, c = (p.Nq + p.G - 1) / p.G;
  for (int b = p.level - 1; b >= 0; --b) {
    if (c <= 1) return;
    const int cL = c >> 1, nL = cL * p.G;
    if ((slot >> b) & 1) {
      start += nL;
      n -= nL;
      c -= cL;
    } else {
      n = nL;
      c = cL;
    }
  }
  if (c <= 1) return;
  const int nL = (c >> 1) * p.G;
  const size_t hbase = (size_t)bh * p.Nq;
  int32_t* nperm = p.perm + hbase + start;
  uint32_t* nkeys = p.keys + hbase + start;
  int32_t* ntmp = p.tmp + hbase + start;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
  const bool gw = w < NB;  // wave owns column block w of C

  // ---- 1. sums and raw scatter --------------------------------------------
  double cacc[NB][16];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) cacc[b][i] = 0.0;
  double ssum = 0.0;
  for (int r0 = 0; r0 < n; r0 += 64) {
    const int rows = min(64, n - r0);
    if constexpr (BF16) {
      __bf16* Xt = (__bf16*)stage_raw;
      const __bf16* Qb = (const __bf16*)p.Q;
      for (int e = tid; e < 64 * (D / 8); e += 256) {
        const int r = e / (D / 8), ch = e % (D / 8);
        bf16x8 v = {};
        if (r < rows) v = *(const bf16x8*)(Qb + (hbase + nperm[r0 + r]) * D + ch * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) Xt[(ch * 8 + j) * XS + r] = v[j];
      }
    } else {
      float* Xs = (float*)stage_raw;
      const float* Qf = (const float*)p.Q;
      for (int e = tid; e < 64 * (D / 4); e += 256) {
        const int r = e / (D / 4), ch = e % (D / 4);
        f32x4 v = {};
        if (r < rows) v = *(const f32x4*)(Qf + (hbase + nperm[r0 + r]) * D + ch * 4);
        *(f32x4*)(Xs + r * FS + ch * 4) = v;
      }
    }
    __syncthreads();
    if (tid < D) {
      if constexpr (BF16) {
        const __bf16* Xt = (const __bf16*)stage_raw;
        for (int r = 0; r < 64; ++r) ssum += (double)(float)Xt[tid * XS + r];
      } else {
        const float* Xs = (const float*)stage_raw;
        for (int r = 0; r < 64; ++r) ssum += (double)Xs[r * FS + tid];
      }
    }
    if (gw) {
      if constexpr (BF16) {
        const __bf16* Xt = (const __bf16*)stage_raw;
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
          f32x16 a32 = {};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 A = *(const bf16x8*)(Xt + (bi * 32 + ln) * XS + ks * 16 + 8 * h);
            const bf16x8 B = *(const bf16x8*)(Xt + (w * 32 + ln) * XS + ks * 16 + 8 * h);
            a32 = mfma_32x32x16(A, B, a32);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) cacc[bi][i] += (double)a32[i];
        }
      } else {
        const float* Xs = (const float*)stage_raw;
        for (int r = 0; r < 64; ++r) {
          const double xc = (double)Xs[r * FS + w * 32 + ln];
#pragma unroll
          for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              cacc[bi][i] = fma((double)Xs[r * FS + bi * 32 + 8 * (i >> 2) + 4 * h + (i & 3)], xc, cacc[bi][i]);
        }
      }
    }
    __syncthreads();
  }

  // ---- 2. centre and power-iterate -----------------------------------------
  if (tid < D) sS[tid] = ssum;
  __syncthreads();
  const double inv_n = 1.0 / (double)n;
  if (gw) {
    const double sc = sS[w * 32 + ln] * inv_n;
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i) cacc[bi][i] -= sS[bi * 32 + 8 * (i >> 2) + 4 * h + (i & 3)] * sc;
  }
  if (tid < D) sV[tid] = 1.0 / sqrt((double)D);
  __syncthreads();
  for (int it = 0; it < p.iters; ++it) {
    double wv = 0.0;
    if (gw) {
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int i = 0; i < 16; ++i) wv = fma(cacc[bi][i], sV[bi * 32 + 8 * (i >> 2) + 4 * h + (i & 3)], wv);
      wv += __shfl_xor(wv, 32, 64);
    }
    const double sq = wave_sum_f64((gw && h == 0) ? wv * wv : 0.0);
    if (l == 0) sRed[w] = sq;
    __syncthreads();
    const double tot = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
    if (tot == 0.0) break;  // degenerate node: keep the current direction
    const double inv = 1.0 / sqrt(tot);
    if (gw && h == 0) sV[w * 32 + ln] = wv * inv;
    __syncthreads();
  }

  // ---- 3. projections -------------------------------------------------------
  {
    const double mv = wave_sum_f64(tid < D ? sS[tid] * inv_n * sV[tid] : 0.0);
    __syncthreads();
    if (l == 0) sRed[w] = mv;
    __syncthreads();
  }
  const double muv = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
  for (int i = tid; i < n; i += 256) {
    const size_t row = (hbase + nperm[i]) * D;
    double dot = 0.0;
    if constexpr (BF16) {
      const __bf16* qp = (const __bf16*)p.Q + row;
#pragma unroll
      for (int ch = 0; ch < D / 8; ++ch) {
        const bf16x8 v = *(const bf16x8*)(qp + ch * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) dot = fma((double)(float)v[j], sV[ch * 8 + j], dot);
      }
    } else {
      const float* qp = (const float*)p.Q + row;
#pragma unroll
      for (int ch = 0; ch < D / 4; ++ch) {
        const f32x4 v = *(const f32x4*)(qp + ch * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) dot = fma((double)v[j], sV[ch * 4 + j], dot);
      }
    }
    const float pf = (float)(dot - muv) + 0.0f;  // + 0 folds -0 into +0
    nkeys[i] = float_order_key(pf);
  }
  __syncthreads();

  // ---- 4. rank select and stable partition ---------------------------------
  uint32_t prefix = 0, pmask = 0;
  int krem = nL;  // rank (from the bottom) still to locate among keys matching prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const uint32_t u = nkeys[i];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    const int cnt = hist[tid];
    const int cum = scan256(cnt, s_wsum);
    if (cum >= krem && cum - cnt < krem) {
      s_prefix = prefix | ((uint32_t)tid << shift);
      s_krem = krem - (cum - cnt);
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    pmask |= 0xFFu << shift;
  }
  const uint32_t T = prefix;
  int base_left = 0, base_tie = 0;
  for (int s0 = 0; s0 < n; s0 += 256) {
    const int i = s0 + tid;
    const bool valid = i < n;
    const uint32_t u = valid ? nkeys[i] : 0xFFFFFFFFu;
    const int lt = (valid && u < T) ? 1 : 0;
    const int eq = (valid && u == T) ? 1 : 0;
    const int tie_incl = scan256(eq, s_wsum);
    const int left = (lt || (eq && base_tie + tie_incl - eq < krem)) ? 1 : 0;
    const int left_incl = scan256(left, s_wsum);
    if (valid) {
      const int lpos = base_left + left_incl - left;
      ntmp[left ? lpos : nL + (i - lpos)] = nperm[i];
    }
    if (tid == 255) {
      s_tot[0] = tie_incl;
      s_tot[1] = left_incl;
    }
    __syncthreads();
    base_tie += s_tot[0];
    base_left += s_tot[1];
    __syncthreads();
  }
  for (int i = tid; i < n; i += 256) nperm[i] = ntmp[i];
}

template <int D, bool BF16>
void launch_levels(const Shape& s, const void* Q, int32_t* perm, int32_t* tmp, uint32_t* keys, hipStream_t st) {
  int levels = 0;
  while ((1 << levels) < s.c) ++levels;
  PddpParams p{Q, perm, tmp, keys, s.Nq, s.G, s.iters, 0};
  for (int lv = 0; lv < levels; ++lv) {
    p.level = lv;
    hipLaunchKernelGGL((pddp_level_kernel<D, BF16>), dim3(1u << lv, s.BH), dim3(256), 0, st, p);
  }
}

}  // namespace

size_t pddp_workspace_bytes(const Shape& s) {
  const size_t n = (size_t)s.BH * s.Nq;
  return ((n * 4 + 255) / 256) * 256 * 2;
}

hipError_t launch_pddp(const Shape& s, bool bf16, const void* Q, int32_t* perm, void* ws, hipStream_t st) {
  const size_t n = (size_t)s.BH * s.Nq;
  int32_t* tmp = (int32_t*)ws;
  uint32_t* keys = (uint32_t*)((char*)ws + ((n * 4 + 255) / 256) * 256);
  hipLaunchKernelGGL(pddp_init_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, perm, s.Nq, n);
  if (bf16) {
    if (s.d == 128) launch_levels<128, true>(s, Q, perm, tmp, keys, st);
    else launch_levels<64, true>(s, Q, perm, tmp, keys, st);
  } else {
    if (s.d == 128) launch_levels<128, false>(s, Q, perm, tmp, keys, st);
    else launch_levels<64, false>(s, Q, perm, tmp, keys, st);
  }
  return hipGetLastError();
}

}  // namespace mcs
