// Residual-drift check for adaptive anchoring.
//
// MC-Sparse review (blog.secrett2633.cloud), section 3: the exact selections
// and the dense-sparse residual taken at an anchor are reused on the next
// steps because the attention pattern and the residual change little from
// step to step.  This measures how far they have moved: exact attention on a
// few sampled query rows, compared with the caller's output for the step.
// For a reuse output O = O_sparse + R_anchor the difference is
// R_anchor - R_now, so drift = ||O - O_exact|| / ||O_exact|| over the sampled
// rows is the residual's movement relative to the output.
//
// Kernels.  rows_partial_*: exact attention of the sampled rows split over
// key ranges (flash-decoding style: each workgroup one (head, key range),
// writing per row the running maximum m in scaled log2 units, the sum l and
// the unnormalised output relative to m); bf16 on MFMA with the per-wave core
// of ring.hpp (4 waves x 32 rows, 64-key K/V tiles by direct-to-LDS copies),
// float32 on the VALU (one wave per row and key range).  drift_combine_kernel:
// per (head, sampled row) the merged exact row and its squared error and norm
// against the caller's output; drift_final_kernel: per head, the sums in row
// order and the ratio.
#include "mcs_kernels.hpp"
#include "ring.hpp"

namespace mcs {
namespace {

constexpr int kDriftTK = 64;  // keys per tile

struct DriftParams {
  const void *Q, *K, *V, *O;
  const int32_t* rows;
  float* pm;     // [BH][nsplit][n_rows][2]: m (scaled log2), l
  float* po;     // [BH][nsplit][n_rows][d]: unnormalised output
  float* perr;   // [BH][n_rows][2]: squared error, squared norm
  float* drift;  // [BH]
  int Nq, Nkv, n_rows, nsplit, tps;
  float c;       // scale * log2(e)
  float scale;
  int causal_block, q_offset;
};

__device__ __forceinline__ int sampled_row(const DriftParams& p, int r) {
  return min(max(p.rows[r], 0), p.Nq - 1);
}

// bf16: workgroup = (head, key range); wave w owns sampled rows 32w..32w+31.
template <int D>
__global__ __launch_bounds__(256) void rows_partial_bf16_kernel(DriftParams p) {
  constexpr int CH = D / 8, RPL = 64 / CH, LPW = kDriftTK / RPL / 4;  // DMA copies per wave per tile
  constexpr int BYTES = kDriftTK * D * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char ks[2][BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vs[2][BYTES];
  const int bh = blockIdx.x / p.nsplit, sp = blockIdx.x - bh * p.nsplit;
  const int w = wave_id(), l = lane_id(), n = l & 31, h = l >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int r = 32 * w + n;
  const bool valid = r < p.n_rows;
  const int row = valid ? sampled_row(p, r) : 0;
  FlashCore<D> fc;
  fc.init((const __bf16*)p.Q + ((size_t)bh * p.Nq + row) * D, valid);
  const int lim = valid ? visible_limit(row, p.causal_block, p.q_offset, p.Nkv) : 0;
  // tiles past every sampled row's visible limit are skipped
  __shared__ int s_lim[4];
  int wl = lim;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wl = max(wl, __shfl_xor(wl, o, 64));
  if (l == 0) s_lim[w] = wl;
  __syncthreads();
  const int kmax = max(max(s_lim[0], s_lim[1]), max(s_lim[2], s_lim[3]));
  const int ntiles = (kmax + kDriftTK - 1) / kDriftTK;
  const int t0 = sp * p.tps, t1 = min(t0 + p.tps, ntiles);
  const __bf16* Kh = (const __bf16*)p.K + (size_t)bh * p.Nkv * D;
  const __bf16* Vh = (const __bf16*)p.V + (size_t)bh * p.Nkv * D;
  int voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int rr = RPL * (wu + 4 * j) + l / CH;
    voff[j] = rr * (2 * D) + (((l % CH) ^ swz<D>(rr)) * 16);
  }
  // rows past the end of the head read as zeros (their keys are masked)
  auto issue = [&](int t, int slot) {
    const int bytes = (p.Nkv - t * kDriftTK) * D * 2;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(Kh + (size_t)t * kDriftTK * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(Vh + (size_t)t * kDriftTK * D, bytes);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      dma16_buf(rk, voff[j], ks[slot] + (wu + 4 * j) * 1024);
      dma16_buf(rv, voff[j], vs[slot] + (wu + 4 * j) * 1024);
    }
  };
  // two-slot ring: tile t + 1 is copied while tile t is used; the slot it
  // overwrites was last read before the previous iteration's final barrier
  if (t0 < t1) issue(t0, 0);
  for (int t = t0; t < t1; ++t) {
    const int slot = (t - t0) & 1;
    if (t + 1 < t1) {
      issue(t + 1, slot ^ 1);
      wait_vmcnt<2 * LPW>();  // tile t landed; t + 1 may still be in flight
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    fc.template blocks<2, 32 * 2 * D>(ks[slot], vs[slot], lim - t * kDriftTK, p.c);
    __syncthreads();
  }
  const float lt = half_sum(fc.l_run);
  if (!valid) return;
  const size_t pr = ((size_t)bh * p.nsplit + sp) * p.n_rows + r;
  if (h == 0) {
    p.pm[2 * pr] = fc.m_run;
    p.pm[2 * pr + 1] = lt;
  }
  float* o = p.po + pr * D;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) *(f32x4*)(o + b * 32 + 8 * q4 + 4 * h) = fc.out4(b, q4, 1.f);
}

// float32: one wave per (head, key range, sampled row); lane j takes keys
// j, j + 64, ... of the range with its own running maximum, then the 64 lanes
// are merged in lane order through LDS.
template <int D>
__global__ __launch_bounds__(64) void rows_partial_f32_kernel(DriftParams p) {
  __shared__ float sq[D];
  __shared__ float sm[64], sl[64];
  __shared__ float so[64][D + 1];
  const int r = blockIdx.x % p.n_rows;
  const int rest = blockIdx.x / p.n_rows;
  const int sp = rest % p.nsplit, bh = rest / p.nsplit;
  const int l = threadIdx.x;
  const int row = sampled_row(p, r);
  const float* Qh = (const float*)p.Q + ((size_t)bh * p.Nq + row) * D;
  for (int e = l; e < D; e += 64) sq[e] = Qh[e];
  __syncthreads();
  const int lim = visible_limit(row, p.causal_block, p.q_offset, p.Nkv);
  const int k0 = sp * p.tps * kDriftTK, k1 = min(min(k0 + p.tps * kDriftTK, p.Nkv), lim);
  const float* Kh = (const float*)p.K + (size_t)bh * p.Nkv * D;
  const float* Vh = (const float*)p.V + (size_t)bh * p.Nkv * D;
  float m = -kInf, s = 0.f, o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) o[e] = 0.f;
  for (int j = k0 + l; j < k1; j += 64) {
    float x = 0.f;
    for (int e = 0; e < D; ++e) x = fmaf(sq[e], Kh[(size_t)j * D + e], x);
    x *= p.c;
    const float mn = fmaxf(m, x);
    const float a = exp2f(m - mn), pj = exp2f(x - mn);
    s = s * a + pj;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = fmaf(o[e], a, pj * Vh[(size_t)j * D + e]);
    m = mn;
  }
  sm[l] = m;
  sl[l] = s;
#pragma unroll
  for (int e = 0; e < D; ++e) so[l][e] = o[e];
  __syncthreads();
  float M = -kInf;
  for (int i = 0; i < 64; ++i) M = fmaxf(M, sm[i]);
  const size_t pr = ((size_t)bh * p.nsplit + sp) * p.n_rows + r;
  if (l == 0) {
    float L = 0.f;
    for (int i = 0; i < 64; ++i)
      if (sm[i] != -kInf) L += sl[i] * exp2f(sm[i] - M);
    p.pm[2 * pr] = M;
    p.pm[2 * pr + 1] = L;
  }
  for (int e = l; e < D; e += 64) {
    float acc = 0.f;
    for (int i = 0; i < 64; ++i)
      if (sm[i] != -kInf) acc += so[i][e] * exp2f(sm[i] - M);
    p.po[pr * D + e] = acc;
  }
}

// Merge the key ranges of one sampled row of one head and compare with the
// caller's output row.  Wave 0 takes one key range per lane (the maximum,
// the weights 2^(m_s - M) and the merged sum, to LDS); then thread ch of the
// first D merges that channel over the ranges, eight loads in flight.
template <typename T, int D>
__global__ __launch_bounds__(256) void drift_combine_kernel(DriftParams p) {
  __shared__ float wgt[kMaxDriftSplits];
  __shared__ float s_L;
  __shared__ float red[2][D];
  const int bh = blockIdx.x / p.n_rows, r = blockIdx.x - bh * p.n_rows;
  const size_t base = (size_t)bh * p.nsplit * p.n_rows + r;  // (bh, split 0, r)
  const int tid = threadIdx.x;
  if (tid < 64) {
    float M = -kInf;
    for (int s = tid; s < p.nsplit; s += 64) M = fmaxf(M, p.pm[2 * (base + (size_t)s * p.n_rows)]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float L = 0.f;
    for (int s = tid; s < p.nsplit; s += 64) {
      const size_t pr = base + (size_t)s * p.n_rows;
      const float ms = p.pm[2 * pr];
      const float wv = (ms == -kInf) ? 0.f : exp2f(ms - M);
      wgt[s] = wv;
      L = fmaf(p.pm[2 * pr + 1], wv, L);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
    if (tid == 0) s_L = L;
  }
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < p.nsplit; ++s) acc = fmaf(p.po[(base + (size_t)s * p.n_rows) * D + tid], wgt[s], acc);
    const float L = s_L;
    const float ex = L > 0.f ? acc / L : 0.f;
    const float got = (float)((const T*)p.O)[((size_t)bh * p.Nq + sampled_row(p, r)) * D + tid];
    const float dlt = got - ex;
    red[0][tid] = dlt * dlt;
    red[1][tid] = ex * ex;
  }
  __syncthreads();
  if (tid == 0) {
    float e2 = 0.f, r2 = 0.f;
    for (int i = 0; i < D; ++i) {
      e2 += red[0][i];
      r2 += red[1][i];
    }
    p.perr[2 * ((size_t)bh * p.n_rows + r)] = e2;
    p.perr[2 * ((size_t)bh * p.n_rows + r) + 1] = r2;
  }
}

// One workgroup for all heads: wave w takes heads w, w + 16, ... (lane i
// adds rows i, i + 64, ... in order, then a fixed butterfly over the lanes);
// then the largest drift over the heads (NaN if any is NaN) goes to
// drift[BH].
__global__ __launch_bounds__(1024) void drift_final_kernel(DriftParams p, int BH) {
  __shared__ float s_max[16];
  const int w = wave_id(), l = lane_id();
  const float qnan = __builtin_nanf("");
  auto mx2 = [&](float x, float y) { return (x != x || y != y) ? qnan : fmaxf(x, y); };
  float mx = 0.f;
  for (int bh = w; bh < BH; bh += 16) {
    float a = 0.f, b = 0.f;
    for (int r = l; r < p.n_rows; r += 64) {
      a += p.perr[2 * ((size_t)bh * p.n_rows + r)];
      b += p.perr[2 * ((size_t)bh * p.n_rows + r) + 1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      a += __shfl_xor(a, o, 64);
      b += __shfl_xor(b, o, 64);
    }
    const float dr = b > 0.f ? sqrtf(a / b) : 0.f;
    if (l == 0) p.drift[bh] = dr;
    mx = mx2(mx, dr);
  }
  if (l == 0) s_max[w] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = 0.f;
    for (int i = 0; i < 16; ++i) m = mx2(m, s_max[i]);
    p.drift[BH] = m;
  }
}

void drift_split(const Shape& s, int& nsplit, int& tps) {
  const int ntiles = (s.Nkv + kDriftTK - 1) / kDriftTK;
  tps = std::max(8, (ntiles + kMaxDriftSplits - 1) / kMaxDriftSplits);
  nsplit = (ntiles + tps - 1) / tps;
}

}  // namespace

size_t drift_workspace_bytes(const Shape& s, int n_rows) {
  int nsplit, tps;
  drift_split(s, nsplit, tps);
  return (size_t)s.BH * ((size_t)nsplit * n_rows * (2 + s.d) + (size_t)n_rows * 2) * 4;
}

hipError_t launch_drift(const Shape& s, bool bf16, const void* Q, const void* K, const void* V, const void* O,
                        const int32_t* rows, int n_rows, float* drift, void* ws, hipStream_t st) {
  DriftParams p;
  p.Q = Q; p.K = K; p.V = V; p.O = O; p.rows = rows; p.drift = drift;
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.n_rows = n_rows;
  drift_split(s, p.nsplit, p.tps);
  p.pm = (float*)ws;
  p.po = p.pm + (size_t)s.BH * p.nsplit * n_rows * 2;
  p.perr = p.po + (size_t)s.BH * p.nsplit * n_rows * s.d;
  p.c = s.scale * kLog2e; p.scale = s.scale;
  p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  const dim3 gpart((unsigned)((long long)s.BH * p.nsplit));
  if (bf16) {
    if (s.d == 128) hipLaunchKernelGGL(rows_partial_bf16_kernel<128>, gpart, dim3(256), 0, st, p);
    else hipLaunchKernelGGL(rows_partial_bf16_kernel<64>, gpart, dim3(256), 0, st, p);
  } else {
    const dim3 g((unsigned)((long long)s.BH * p.nsplit * n_rows));
    if (s.d == 128) hipLaunchKernelGGL(rows_partial_f32_kernel<128>, g, dim3(64), 0, st, p);
    else hipLaunchKernelGGL(rows_partial_f32_kernel<64>, g, dim3(64), 0, st, p);
  }
  const dim3 gcomb((unsigned)((long long)s.BH * n_rows));
  if (bf16 && s.d == 128) hipLaunchKernelGGL((drift_combine_kernel<__bf16, 128>), gcomb, dim3(256), 0, st, p);
  else if (bf16) hipLaunchKernelGGL((drift_combine_kernel<__bf16, 64>), gcomb, dim3(256), 0, st, p);
  else if (s.d == 128) hipLaunchKernelGGL((drift_combine_kernel<float, 128>), gcomb, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((drift_combine_kernel<float, 64>), gcomb, dim3(256), 0, st, p);
  hipLaunchKernelGGL(drift_final_kernel, dim3(1), dim3(1024), 0, st, p, s.BH);
  return hipGetLastError();
}

}  // namespace mcs
