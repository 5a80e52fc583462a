// Single-pass anchor selection for bf16: each group's exact column mass is
// kept in LDS and its top-k is selected by the same workgroup, without the
// mass matrix in memory.
//
// Method: MC-Sparse review (blog.secrett2633.cloud), section "3. Method & Key
// Results": at an anchor step each query group keeps the individual KV tokens
// of largest exact attention score, here the column mass
//   m_g[j] = sum_{i in g} exp(scale*<q_i,k_j> - lse_i)   (0 if not visible).
//
// One workgroup (four waves) per (head, group).  Keys past the launch's
// visible limit kv (the last query's limit; Nkv without a causal mask) have
// mass 0 for every group, so the row is kept only for [0, kv): kv*4 bytes of
// LDS (at most 131072, i.e. kv <= 32768).  Phase 1: the waves take the
// visible 32-key blocks in turn; each wave holds 64 queries as two 32-row
// MFMA blocks (S = Q K^T, a lane owns one key column) and reads the K operand
// of a block straight from global memory (the rows stay in L1/L2 for the
// group's other operand reads), one block ahead of its use.  For G = 64 all
// waves hold the group's queries and every key's mass is written once; for
// G = 128 waves 2i and 2i+1 hold the two query halves of the same key blocks
// and add their sums into the zero-initialised row (two addends: the order
// cannot change the sum).  The per-key arithmetic (exponentials, mask, the
// order of the sums) is the column-mass kernel's, so the masses equal those
// of the two-pass anchor bit for bit.  Phase 2: the block select of
// select.hpp over the row in LDS (keys re-read from LDS on every pass)
// finds the min(k, kv) largest masses, equal masses lowest index first; when
// k > kv the zero-mass keys kv, kv+1, ... complete the selection, as the
// tie rule of a full-length row would take them.
#include "mcs_kernels.hpp"
#include "ring.hpp"
#include "select.hpp"

namespace mcs {
namespace {

constexpr int kFusedThreads = 256;
constexpr int kFusedBlk = 32;  // keys per block

struct FusedParams {
  const __bf16 *Q, *K;
  const int32_t* perm;
  const float* lse;  // natural log, [BH][Nq]
  int32_t* idx;      // [BH][c][k]
  int Nq, Nkv, c, k, kv, n_units, per_xcd;
  float c_log2;
  int causal_block, q_offset;
};

struct LdsMassKeys {
  const uint32_t* row;
  __device__ __forceinline__ uint32_t operator()(int j) const {
    const uint32_t u = row[j];
    return (u & 0x80000000u) ? 0u : u;
  }
};

template <int D, int G>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void anchor_fused_bf16_kernel(FusedParams p) {
  constexpr int NKS = D / 16, NW = kFusedThreads / 64;
  constexpr int QH = G / 64;        // query halves of 64 (waves holding different queries)
  constexpr int KSTRIDE = NW / QH;  // waves sharing one query half take every KSTRIDE-th block
  using Sel = BlockSelect<kFusedThreads, 0>;
  __shared__ typename Sel::Shared sh;
  __shared__ __attribute__((aligned(16))) float s_lse[G];
  __shared__ __attribute__((aligned(16))) int s_lim[G];
  __shared__ int s_kmax[NW];
  extern __shared__ __attribute__((aligned(16))) float s_mass[];  // [kv]

  const int unit = xcd_unit(blockIdx.x, p.per_xcd);
  if (unit >= p.n_units) return;
  const int bh = unit / p.c, g = unit - bh * p.c;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n = l & 31, h = l >> 5;
  const int qh = w % QH, ks0 = w / QH;  // this wave's query half and first key block
  const int gsize = min(G, p.Nq - g * G);
  const int32_t* gperm = p.perm + (size_t)bh * p.Nq + (size_t)g * G;

  for (int j = tid; j < p.kv; j += kFusedThreads) s_mass[j] = 0.f;
  // per query of the group: lse in base 2 (+inf for padding rows so they add 0) and its limit
  for (int i = tid; i < G; i += kFusedThreads) {
    const bool v = i < gsize;
    const int row = v ? min(max(gperm[i], 0), p.Nq - 1) : 0;
    const float ls = p.lse[(size_t)bh * p.Nq + row];
    s_lse[i] = (!v || ls == -kInf) ? kInf : ls * kLog2e;
    s_lim[i] = v ? visible_limit(row, p.causal_block, p.q_offset, p.Nkv) : 0;
  }
  // this wave's 64 queries (query half qh) as two 32-row A operands
  bf16x8 qa[2][NKS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = 64 * qh + 32 * qb + n;
    const bool v = i < gsize;
    const int row = v ? min(max(gperm[i], 0), p.Nq - 1) : 0;
    const __bf16* qp = p.Q + ((size_t)bh * p.Nq + row) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 z = {};
      qa[qb][ks] = v ? *(const bf16x8*)(qp + ks * 16) : z;
    }
  }
  __syncthreads();
  // score row i of block qb on this lane: query 64 qh + 32 qb + 8 (i/4) + 4 h + i%4
  float lse2[2][16];
  int lmin = p.Nkv, lmax = 0;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q0 = 64 * qh + 32 * qb + 8 * r + 4 * h;
      const f32x4 v4 = *(const f32x4*)&s_lse[q0];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lse2[qb][4 * r + e] = v4[e];
        if (q0 + e < gsize) {
          lmin = min(lmin, s_lim[q0 + e]);
          lmax = max(lmax, s_lim[q0 + e]);
        }
      }
    }
  lmin = min(lmin, __shfl_xor(lmin, 32, 64));
  lmax = max(lmax, __shfl_xor(lmax, 32, 64));
  // the whole group's largest limit: every wave covers the key blocks any of its queries sees
  if (l == 0) s_kmax[w] = lmax;
  __syncthreads();
  int kmax = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) kmax = max(kmax, s_kmax[i]);
  const int nblk = (min(kmax, p.kv) + kFusedBlk - 1) / kFusedBlk;

  // K operand of key block b: lane (n, h) holds key 32 b + n, channels 16 ks + 8 h + 0..7
  // (rows past the end of the head read as zeros through the buffer range; their keys are masked)
  const __amdgpu_buffer_rsrc_t kres = buffer_rsrc(p.K + (size_t)bh * p.Nkv * D, p.Nkv * D * 2);
  auto load_k = [&](int b, bf16x8 (&kk)[NKS]) {
    const int off = ((b * kFusedBlk + n) * D + 8 * h) * 2;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kk[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kres, off + 32 * ks, 0, 0));
  };
  bf16x8 kn[NKS];
  int b = ks0;
  if (b < nblk) load_k(b, kn);
  for (; b < nblk; b += KSTRIDE) {
    bf16x8 kk[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kk[ks] = kn[ks];
    if (b + KSTRIDE < nblk) load_k(b + KSTRIDE, kn);
    f32x16 s[2] = {};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      s[0] = mfma_32x32x16(qa[0][ks], kk[ks], s[0]);
      s[1] = mfma_32x32x16(qa[1][ks], kk[ks], s[1]);
    }
    const int key = b * kFusedBlk + n;
    float cs = 0.f;
    if (b * kFusedBlk + kFusedBlk <= lmin) {  // every key of the block visible to every query of the wave
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) cs += fast_exp2(fmaf(s[qb][i], p.c_log2, -lse2[qb][i]));
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q0 = 64 * qh + 32 * qb + 8 * r + 4 * h;
          const int4 lm = *(const int4*)&s_lim[q0];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = fast_exp2(fmaf(s[qb][4 * r + e], p.c_log2, -lse2[qb][4 * r + e]));
            cs += (key < lm[e]) ? pv : 0.f;
          }
        }
    }
    const float m = half_sum(cs);  // the wave's 64 queries
    if (h == 0 && key < p.kv) {
      if constexpr (QH == 1) s_mass[key] = m;
      else atomicAdd(&s_mass[key], m);
    }
  }
  __syncthreads();

  // phase 2: the selection over the row in LDS
  int32_t* out = p.idx + ((size_t)bh * p.c + g) * p.k;
  const LdsMassKeys keys{(const uint32_t*)s_mass};
  const int need = min(p.k, p.kv);
  Sel sel;
  sel.n = p.kv;
  uint32_t T;
  int tie_need;
  sel.template threshold<31>(keys, need, sh, T, tie_need);
  sel.split(keys, T, tie_need, sh, [&](int, int j, bool sl, int pos) {
    if (sl && pos < need) out[pos] = j;
  });
  for (int i = p.kv + tid; i < p.k; i += kFusedThreads) out[i] = i;  // zero-mass keys past the visible limit
}

template <int D, int G>
void launch_fused(const FusedParams& p, dim3 grid, size_t lds, hipStream_t st) {
  static const bool attr = allow_dynamic_lds((const void*)anchor_fused_bf16_kernel<D, G>, kFusedMaxKv * 4);
  (void)attr;
  hipLaunchKernelGGL((anchor_fused_bf16_kernel<D, G>), grid, dim3(kFusedThreads), lds, st, p);
}

}  // namespace

int fused_anchor_row(const Shape& s) {
  if (!s.causal_block || s.Nq < 1) return s.Nkv;
  const long long lim = ((long long)(s.q_offset + s.Nq - 1) / s.causal_block + 1) * s.causal_block;
  return lim < s.Nkv ? (int)lim : s.Nkv;
}

hipError_t launch_anchor_fused_bf16(const Shape& s, const void* Q, const void* K, const int32_t* perm,
                                    const float* lse, int32_t* idx, hipStream_t st) {
  FusedParams p;
  p.Q = (const __bf16*)Q; p.K = (const __bf16*)K; p.perm = perm; p.lse = lse; p.idx = idx;
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.c = s.c; p.k = s.k; p.kv = fused_anchor_row(s);
  p.c_log2 = s.scale * kLog2e; p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  p.n_units = s.BH * s.c;
  p.per_xcd = (p.n_units + 7) / 8;
  const dim3 grid(8 * p.per_xcd);
  const size_t lds = ((size_t)p.kv * 4 + 15) / 16 * 16;
  if (s.d == 128 && s.G == 64) launch_fused<128, 64>(p, grid, lds, st);
  else if (s.d == 128) launch_fused<128, 128>(p, grid, lds, st);
  else if (s.G == 64) launch_fused<64, 64>(p, grid, lds, st);
  else launch_fused<64, 128>(p, grid, lds, st);
  return hipGetLastError();
}

}  // namespace mcs
