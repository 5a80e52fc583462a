// float32 path of the attention kernels (small problems; no MFMA).  One
// thread per query row (dense, sparse) or per key (mass).  Logits and
// softmax normalisers are accumulated in float64 so that the selection made
// from the column mass is as exact as the inputs allow.
//
// Same operations as the bf16 kernels: exact dense attention, per-group
// column mass and gathered sparse attention with the residual, as described
// in the MC-Sparse review (blog.secrett2633.cloud), section 3.
#include "mcs_device.hpp"
#include "mcs_kernels.hpp"

namespace mcs {
namespace {

struct F32Params {
  const float *Q, *K, *V;
  const int32_t *perm, *idx;
  const float* lse_in;
  float *O, *lse, *Ofull, *R, *mass;
  int Nq, Nkv, k, c, G, bh0;
  double scale;
  int causal_block, q_offset, anchor;
};

// Online softmax over a list of keys for one query row held in registers.
template <int D, typename KeyAt>
__device__ __forceinline__ void attend_row(const float* q, const float* Kh, const float* Vh, int nkeys,
                                           KeyAt key_at, double scale, float* o, double& m, double& l) {
  m = -__builtin_huge_val();
  l = 0.0;
#pragma unroll
  for (int i = 0; i < D; ++i) o[i] = 0.f;
  for (int t = 0; t < nkeys; ++t) {
    const int j = key_at(t);
    const float* kp = Kh + (size_t)j * D;
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < D; ++i) s = fma((double)q[i], (double)kp[i], s);
    s *= scale;
    if (s > m) {
      const float alpha = (float)exp(m - s);
      l *= exp(m - s);
#pragma unroll
      for (int i = 0; i < D; ++i) o[i] *= alpha;
      m = s;
    }
    const double pw = exp(s - m);
    l += pw;
    const float pf = (float)pw;
    const float* vp = Vh + (size_t)j * D;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] = fmaf(pf, vp[i], o[i]);
  }
}

template <int D>
__global__ __launch_bounds__(64) void dense_f32_kernel(F32Params p) {
  const int bh = blockIdx.y;
  const int q = blockIdx.x * 64 + threadIdx.x;
  if (q >= p.Nq) return;
  float qv[D], o[D];
  const float* qp = p.Q + ((size_t)bh * p.Nq + q) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) qv[i] = qp[i];
  double m, l;
  const int nk = visible_limit(q, p.causal_block, p.q_offset, p.Nkv);
  attend_row<D>(qv, p.K + (size_t)bh * p.Nkv * D, p.V + (size_t)bh * p.Nkv * D, nk,
                [](int t) { return t; }, p.scale, o, m, l);
  const float inv = l > 0.0 ? (float)(1.0 / l) : 0.f;
  const size_t row = (size_t)bh * p.Nq + q;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    p.O[row * D + i] = o[i] * inv;
    if (p.Ofull) p.Ofull[row * D + i] = o[i] * inv;
  }
  if (p.lse) p.lse[row] = l > 0.0 ? (float)(m + log(l)) : -__builtin_huge_valf();
}

template <int D>
__global__ __launch_bounds__(128) void sparse_f32_kernel(F32Params p) {
  const int bh = blockIdx.y, g = blockIdx.x;
  const int r = threadIdx.x;
  const int gsize = min(p.G, p.Nq - g * p.G);
  if (r >= gsize) return;
  const int q = min(max(p.perm[(size_t)bh * p.Nq + (size_t)g * p.G + r], 0), p.Nq - 1);
  const int32_t* sel = p.idx + ((size_t)bh * p.c + g) * p.k;
  int nk = p.k;
  if (p.causal_block) {
    const int lim = visible_limit(q, p.causal_block, p.q_offset, p.Nkv);
    int lo = 0, hi = p.k;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sel[mid] < lim) lo = mid + 1; else hi = mid;
    }
    nk = lo;
  }
  float qv[D], o[D];
  const float* qp = p.Q + ((size_t)bh * p.Nq + q) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) qv[i] = qp[i];
  double m, l;
  attend_row<D>(qv, p.K + (size_t)bh * p.Nkv * D, p.V + (size_t)bh * p.Nkv * D, nk,
                [sel, &p](int t) { return min(max(sel[t], 0), p.Nkv - 1); }, p.scale, o, m, l);
  const float inv = l > 0.0 ? (float)(1.0 / l) : 0.f;
  const size_t row = (size_t)bh * p.Nq + q;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const float v = o[i] * inv;
    if (p.anchor) p.R[row * D + i] -= v;
    else p.O[row * D + i] = v + (p.R ? p.R[row * D + i] : 0.f);
  }
}

// mass[(bh-bh0)*c + g][j]: one workgroup per (group, head); the group's query
// rows and their lse are staged in LDS, each thread owns keys.
template <int D>
__global__ __launch_bounds__(256) void mass_f32_kernel(F32Params p) {
  __shared__ float sq[128 * D];
  __shared__ double slse[128];
  __shared__ int slim[128];
  const int bhl = blockIdx.y, bh = p.bh0 + bhl, g = blockIdx.x;
  const int gsize = min(p.G, p.Nq - g * p.G);
  for (int e = threadIdx.x; e < gsize * D; e += 256) {
    const int r = e / D, i = e % D;
    const int q = min(max(p.perm[(size_t)bh * p.Nq + (size_t)g * p.G + r], 0), p.Nq - 1);
    sq[e] = p.Q[((size_t)bh * p.Nq + q) * D + i];
    if (i == 0) {
      slse[r] = (double)p.lse_in[(size_t)bh * p.Nq + q];
      slim[r] = visible_limit(q, p.causal_block, p.q_offset, p.Nkv);
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < p.Nkv; j += 256) {
    float kv[D];
    const float* kp = p.K + ((size_t)bh * p.Nkv + j) * D;
#pragma unroll
    for (int i = 0; i < D; ++i) kv[i] = kp[i];
    double m = 0.0;
    for (int r = 0; r < gsize; ++r) {
      if (j >= slim[r] || slse[r] == -__builtin_huge_val()) continue;
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < D; ++i) s = fma((double)sq[r * D + i], (double)kv[i], s);
      m += exp(s * p.scale - slse[r]);
    }
    p.mass[((size_t)bhl * p.c + g) * p.Nkv + j] = (float)m;
  }
}

}  // namespace

hipError_t launch_dense_f32(const Shape& s, const void* Q, const void* K, const void* V, void* O,
                            float* lse, float* Ofull, hipStream_t st) {
  F32Params p = {};
  p.Q = (const float*)Q; p.K = (const float*)K; p.V = (const float*)V;
  p.O = (float*)O; p.lse = lse; p.Ofull = Ofull;
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.scale = s.scale; p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  const dim3 grid((s.Nq + 63) / 64, s.BH);
  if (s.d == 128) hipLaunchKernelGGL(dense_f32_kernel<128>, grid, dim3(64), 0, st, p);
  else hipLaunchKernelGGL(dense_f32_kernel<64>, grid, dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_sparse_f32(const Shape& s, const void* Q, const void* K, const void* V,
                             const int32_t* perm, const int32_t* idx, float* R, void* O, bool anchor,
                             hipStream_t st) {
  F32Params p = {};
  p.Q = (const float*)Q; p.K = (const float*)K; p.V = (const float*)V;
  p.perm = perm; p.idx = idx; p.R = R; p.O = (float*)O;
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.k = s.k; p.c = s.c; p.G = s.G; p.scale = s.scale;
  p.causal_block = s.causal_block; p.q_offset = s.q_offset; p.anchor = anchor ? 1 : 0;
  const dim3 grid(s.c, s.BH);
  if (s.d == 128) hipLaunchKernelGGL(sparse_f32_kernel<128>, grid, dim3(128), 0, st, p);
  else hipLaunchKernelGGL(sparse_f32_kernel<64>, grid, dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_mass_f32(const Shape& s, int bh0, int nbh, const void* Q, const void* K,
                           const int32_t* perm, const float* lse, float* mass, hipStream_t st) {
  F32Params p = {};
  p.Q = (const float*)Q; p.K = (const float*)K; p.perm = perm; p.lse_in = lse; p.mass = mass;
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.c = s.c; p.G = s.G; p.bh0 = bh0; p.scale = s.scale;
  p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  const dim3 grid(s.c, nbh);
  if (s.d == 128) hipLaunchKernelGGL(mass_f32_kernel<128>, grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(mass_f32_kernel<64>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mcs
