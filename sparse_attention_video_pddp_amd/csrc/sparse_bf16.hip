// Gathered sparse attention with the residual (reuse step and anchor
// epilogue) for bf16 on gfx950.
//
// Method: MC-Sparse review (blog.secrett2633.cloud), section "3. Method & Key
// Results": each query group attends only to its own selection of individual
// KV tokens; on reuse steps the anchor's residual R = O_full - O_sparse is
// added back, at the anchor R is formed.
//
// One workgroup owns one (head, group): G/32 waves, 32 query columns each.
// The group's selected K/V rows are gathered in tiles of 32 keys by
// direct-to-LDS loads into a two-slot ring (ring.hpp): tile t+1 is in flight
// while tile t is consumed, with one barrier per tile.  The two slots are
// distinct LDS objects and the loop is unrolled by two, so the compiler can
// tell the slot being read from the slot being filled and adds no wait for
// the in-flight tile.
#include "mcs_kernels.hpp"
#include "ring.hpp"

namespace mcs {
namespace {

template <int D, int G>
struct SparseCfg {
  static constexpr int NW = G / 32;
  static constexpr int NT = 64 * NW;
  static constexpr int TK = 32;                          // keys per tile
  static constexpr int CH = D / 8;                       // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 64 / CH;          // rows filled by one wave-wide load
  static constexpr int LOADS_PER_TENSOR = TK / ROWS_PER_LOAD;
  static constexpr int LOADS_PER_WAVE = LOADS_PER_TENSOR / NW;  // per tensor
  static constexpr int TENSOR_BYTES = TK * D * 2;
  static constexpr int SLOT_BYTES = 2 * TENSOR_BYTES;
  static_assert(LOADS_PER_WAVE >= 1 && LOADS_PER_TENSOR % NW == 0, "load split");
};

struct Params {
  const __bf16 *Q, *K, *V;
  const int32_t *perm, *idx;
  float* R;
  __bf16* O;
  int Nq, Nkv, k, c, n_units, per_xcd;
  float c_log2;
  int causal_block, q_offset;
  int anchor;
};

template <int D, int G>
__global__ __launch_bounds__(2 * G) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_ring_kernel(Params p) {
  using C = SparseCfg<D, G>;
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[C::SLOT_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[C::SLOT_BYTES];
  extern __shared__ __attribute__((aligned(16))) int s_idx[];
  __shared__ int s_kmax[C::NW];

  const int unit = xcd_unit(blockIdx.x, p.per_xcd);
  if (unit >= p.n_units) return;
  const int bh = unit / p.c, g = unit - bh * p.c;
  const int w = wave_id(), l = lane_id(), n = l & 31;
  const int klast = p.Nkv - 1;
  {
    const int32_t* gidx = p.idx + ((size_t)bh * p.c + g) * p.k;
    for (int i = threadIdx.x; i < p.k; i += C::NT) s_idx[i] = min(max(gidx[i], 0), klast);
  }
  const int gsize = min(G, p.Nq - g * G);
  const int qloc = w * 32 + n;
  const bool qv = qloc < gsize;
  const int32_t* gperm = p.perm + (size_t)bh * p.Nq + (size_t)g * G;
  // caller data is not validated on the device; clamping keeps every access in bounds
  const int qrow = min(max(gperm[qv ? qloc : 0], 0), p.Nq - 1);
  __syncthreads();

  // number of selected keys visible to this lane's query (a prefix: ascending list)
  int vcount = qv ? p.k : 0;
  if (qv && p.causal_block) {
    const long long lim64 = ((long long)(p.q_offset + qrow) / p.causal_block + 1) * p.causal_block;
    const int lim = lim64 < p.Nkv ? (int)lim64 : p.Nkv;
    int lo = 0, hi = p.k;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_idx[mid] < lim) lo = mid + 1; else hi = mid;
    }
    vcount = lo;
  }
  int vm = vcount;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) vm = max(vm, __shfl_xor(vm, o, 64));
  if (l == 0) s_kmax[w] = vm;

  FlashCore<D> st;
  st.init(p.Q + ((size_t)bh * p.Nq + qrow) * D, qv);
  __syncthreads();
  int kmax = 0;
#pragma unroll
  for (int i = 0; i < C::NW; ++i) kmax = max(kmax, s_kmax[i]);
  const int ntiles = (kmax + C::TK - 1) / C::TK;

  const __bf16* Kh = p.K + (size_t)bh * p.Nkv * D;
  const __bf16* Vh = p.V + (size_t)bh * p.Nkv * D;
  // this lane's part of every tile load: row r = ROWS_PER_LOAD*(w + NW*j) + l/CH, chunk l%CH
  const int lrow0 = l / C::CH, lchunk = l % C::CH;
  auto issue = [&](int t, unsigned char* slot) {
    const int base = t * C::TK;
#pragma unroll
    for (int j = 0; j < C::LOADS_PER_WAVE; ++j) {
      const int li = w + C::NW * j;
      const int r = C::ROWS_PER_LOAD * li + lrow0;
      const int key = s_idx[min(base + r, p.k - 1)];
      const size_t off = (size_t)key * D + ((lchunk ^ swz<D>(r)) * 8);
      dma16(Kh + off, slot + li * 1024);
      dma16(Vh + off, slot + C::TENSOR_BYTES + li * 1024);
    }
  };
  auto compute = [&](int t, const unsigned char* slot) {
    st.template blocks<1, 0>(slot, slot + C::TENSOR_BYTES, vcount - t * C::TK, p.c_log2);
  };

  if (ntiles > 0) issue(0, slot0);
  for (int t = 0; t < ntiles; t += 2) {
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 1 < ntiles) issue(t + 1, slot1);
    compute(t, slot0);
    if (t + 1 >= ntiles) break;
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 2 < ntiles) issue(t + 2, slot0);
    compute(t + 1, slot1);
  }

  float lse;
  const float inv = st.finish(lse);
  if (qv) {
    const int h = l >> 5;
    const size_t row = ((size_t)bh * p.Nq + qrow) * D;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = b * 32 + 8 * q4 + 4 * h;
        f32x4 v = st.out4(b, q4, inv);
        if (p.anchor) {
          float* rp = p.R + row + d0;
          *(f32x4*)rp = *(const f32x4*)rp - v;
        } else {
          if (p.R) v += *(const f32x4*)(p.R + row + d0);
          bf16x4 o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
          *(bf16x4*)(p.O + row + d0) = o;
        }
      }
  }
}

template <int D, int G>
void launch_ring(const Params& p, dim3 grid, int k, hipStream_t st) {
  using C = SparseCfg<D, G>;
  const size_t lds = (size_t)k * 4;
  static const bool attr = allow_dynamic_lds((const void*)sparse_ring_kernel<D, G>,
                                             160 * 1024 - 2 * C::SLOT_BYTES - 1024);
  (void)attr;
  hipLaunchKernelGGL((sparse_ring_kernel<D, G>), grid, dim3(C::NT), lds, st, p);
}

}  // namespace

hipError_t launch_sparse_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                              const int32_t* perm, const int32_t* idx, float* R, void* O, bool anchor,
                              hipStream_t st) {
  Params p;
  p.Q = (const __bf16*)Q; p.K = (const __bf16*)K; p.V = (const __bf16*)V;
  p.perm = perm; p.idx = idx; p.R = R; p.O = (__bf16*)O;
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.k = s.k; p.c = s.c;
  p.c_log2 = s.scale * kLog2e; p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  p.anchor = anchor ? 1 : 0;
  p.n_units = s.BH * s.c;
  p.per_xcd = (p.n_units + 7) / 8;
  const dim3 grid(8 * p.per_xcd);
  if (s.d == 128 && s.G == 64) launch_ring<128, 64>(p, grid, s.k, st);
  else if (s.d == 128) launch_ring<128, 128>(p, grid, s.k, st);
  else if (s.G == 64) launch_ring<64, 64>(p, grid, s.k, st);
  else launch_ring<64, 128>(p, grid, s.k, st);
  return hipGetLastError();
}

}  // namespace mcs
