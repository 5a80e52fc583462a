// Token-level top-k selection per query group (MC-Sparse review,
// blog.secrett2633.cloud, section 3: each group keeps individual KV tokens
// chosen by their exact attention score).
//
// One workgroup per group row of the mass matrix.  The masses are
// non-negative floats, so their bit patterns order like the values; an exact
// 4-pass MSB-first radix select (8-bit digits, LDS histograms) finds the k-th
// largest pattern T, then one ordered pass keeps every key above T and the
// lowest-index keys equal to T until k are kept.  Keys are emitted in
// ascending index order.  Rows that fit are cached in LDS once.
#include "mcs_device.hpp"
#include "mcs_kernels.hpp"

namespace mcs {
namespace {

constexpr int kTopkRowLds = 36864;  // rows up to this many keys are cached in LDS

struct TopkParams {
  const float* mass;
  int32_t* idx;
  int Nkv, k, c, bh0;
};

// Inclusive scan over a 256-thread block (two barriers).
__device__ __forceinline__ int block_incl_scan256(int v, int* s_wsum) {
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

template <bool IN_LDS>
__global__ __launch_bounds__(256) void topk_kernel(TopkParams p) {
  extern __shared__ uint32_t s_row[];
  __shared__ int hist[256];
  __shared__ int s_wsum[4];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;
  __shared__ int s_tot[2];
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int bhl = unit / p.c, g = unit - bhl * p.c;
  const uint32_t* src = (const uint32_t*)(p.mass + (size_t)unit * p.Nkv);
  int32_t* out = p.idx + ((size_t)(p.bh0 + bhl) * p.c + g) * p.k;
  if constexpr (IN_LDS) {
    for (int j = tid; j < p.Nkv; j += 256) s_row[j] = src[j];
    __syncthreads();
    src = s_row;
  }
  uint32_t prefix = 0, pmask = 0;
  int krem = p.k;  // rank (from the top) still to locate among keys matching prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < p.Nkv; j += 256) {
      const uint32_t u = src[j];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    const int cnt = hist[255 - tid];  // digits in descending order
    const int cum = block_incl_scan256(cnt, s_wsum);
    if (cum >= krem && cum - cnt < krem) {
      s_prefix = prefix | ((uint32_t)(255 - tid) << shift);
      s_krem = krem - (cum - cnt);
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    pmask |= 0xFFu << shift;
  }
  const uint32_t T = prefix;
  const int need = krem;  // keys equal to T that are kept, lowest index first
  int base_sel = 0, base_tie = 0;
  for (int s0 = 0; s0 < p.Nkv && base_sel < p.k; s0 += 256) {
    const int j = s0 + tid;
    const uint32_t u = j < p.Nkv ? src[j] : 0u;
    const int gt = (j < p.Nkv && u > T) ? 1 : 0;
    const int eq = (j < p.Nkv && u == T) ? 1 : 0;
    const int tie_incl = block_incl_scan256(eq, s_wsum);
    const int sel = (gt || (eq && base_tie + tie_incl - eq < need)) ? 1 : 0;
    const int sel_incl = block_incl_scan256(sel, s_wsum);
    if (sel && base_sel + sel_incl <= p.k) out[base_sel + sel_incl - 1] = j;
    if (tid == 255) {
      s_tot[0] = tie_incl;
      s_tot[1] = sel_incl;
    }
    __syncthreads();
    base_tie += s_tot[0];
    base_sel += s_tot[1];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_topk(const Shape& s, int bh0, int nbh, const float* mass, int32_t* idx, hipStream_t st) {
  TopkParams p{mass, idx, s.Nkv, s.k, s.c, bh0};
  const dim3 grid(nbh * s.c);
  if (s.Nkv <= kTopkRowLds) {
    static const bool attr = allow_dynamic_lds((const void*)topk_kernel<true>, kTopkRowLds * 4);
    (void)attr;
    hipLaunchKernelGGL(topk_kernel<true>, grid, dim3(256), (size_t)s.Nkv * 4, st, p);
  }
  else
    hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mcs
