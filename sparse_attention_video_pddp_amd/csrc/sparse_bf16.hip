// Gathered sparse attention with the residual (reuse step and anchor
// epilogue) for bf16 on gfx950.
//
// Method: MC-Sparse review (blog.secrett2633.cloud), section "3. Method & Key
// Results": each query group attends only to its own selection of individual
// KV tokens; on reuse steps the anchor's residual R = O_full - O_sparse is
// added back, at the anchor R is formed.
//
// One workgroup owns one (head, group): G/32 waves, 32 query columns each.
// The selected K/V rows are gathered in tiles of 32 keys by direct-to-LDS
// loads (global_load_lds_dwordx4: no staging registers, no LDS stores) into
// an S-slot ring, so S-1 tiles are in flight while one is consumed, with one
// barrier per tile.  Rows are stored unpadded with a 16-byte-chunk XOR
// swizzle that keeps both the K operand reads (16 rows x 16 B) and the
// transposing V reads (4 rows x 32 B) free of bank conflicts.  Compute per
// tile: S^T = K Q^T (v_mfma_f32_32x32x16_bf16, a lane owns one query
// column), base-2 online softmax with lazy rescaling, O^T += V^T P^T with V^T
// from ds_read_b64_tr_b16.
#include "mcs_device.hpp"
#include "mcs_kernels.hpp"

namespace mcs {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kSlack = 8.0f;  // lazy-rescale threshold, log2 units

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D, int G, int S>
struct Cfg {
  static constexpr int NW = G / 32;
  static constexpr int NT = 64 * NW;
  static constexpr int TK = 32;                          // keys per tile
  static constexpr int CH = D / 8;                       // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 64 / CH;          // rows filled by one wave-wide load
  static constexpr int LOADS_PER_TENSOR = TK / ROWS_PER_LOAD;
  static constexpr int LOADS_PER_WAVE = LOADS_PER_TENSOR / NW;  // per tensor
  static constexpr int TENSOR_BYTES = TK * D * 2;
  static constexpr int SLOT_BYTES = 2 * TENSOR_BYTES;
  static constexpr int RING_BYTES = S * SLOT_BYTES;
  static_assert(LOADS_PER_WAVE >= 1 && LOADS_PER_TENSOR % NW == 0, "load split");
};

// 16-byte chunk c of row r sits at chunk c ^ swz(r) of the LDS row.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 2 * (r & 7) + ((r >> 3) & 1);
  else return 2 * (r & 3) + ((r >> 2) & 1);
}

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

template <int D, int G, int S>
__global__ __launch_bounds__(2 * G) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_ring_kernel(Params p) {
  using C = Cfg<D, G, S>;
  constexpr int NB = D / 32, NKS = D / 16;
  // Ring slots are distinct LDS objects so that the compiler can tell a
  // slot being read from the slot an in-flight direct-to-LDS load targets.
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[C::SLOT_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[C::SLOT_BYTES];
  extern __shared__ __attribute__((aligned(16))) int s_idx[];
  __shared__ int s_kmax[C::NW];

  const int unit = xcd_unit(blockIdx.x, p.per_xcd);
  if (unit >= p.n_units) return;
  const int bh = unit / p.c, g = unit - bh * p.c;
  const int w = wave_id(), l = lane_id(), n = l & 31, h = l >> 5;
  const int klast = p.Nkv - 1;
  {
    const int32_t* gidx = p.idx + ((size_t)bh * p.c + g) * p.k;
    for (int i = threadIdx.x; i < p.k; i += C::NT) s_idx[i] = min(max(gidx[i], 0), klast);
  }
  const int gsize = min(G, p.Nq - g * G);
  const int qloc = w * 32 + n;
  const bool qv = qloc < gsize;
  const int32_t* gperm = p.perm + (size_t)bh * p.Nq + (size_t)g * G;
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

  // Q^T operand (B of S^T = K Q^T): lane holds query n, channels 16*ks + 8*h .. +7
  bf16x8 qb[NKS];
  {
    const __bf16* qp = p.Q + ((size_t)bh * p.Nq + qrow) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 z = {};
      qb[ks] = qv ? *(const bf16x8*)(qp + ks * 16) : z;
    }
  }
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
      __builtin_amdgcn_global_load_lds((const void*)(Kh + off), (lds_void_t*)(slot + li * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(Vh + off),
                                       (lds_void_t*)(slot + C::TENSOR_BYTES + li * 1024), 16, 0, 0);
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
  float m_run = -kInf, l_run = 0.f;
  const float cl = p.c_log2;

  auto compute = [&](int t, const unsigned char* slot) {
    const __bf16* Ks = (const __bf16*)slot;
    const __bf16* Vs = (const __bf16*)(slot + C::TENSOR_BYTES);
    // S^T block: 32 keys x 32 queries
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int cch = 2 * ks + h;
      const bf16x8 a = *(const bf16x8*)(Ks + n * D + ((cch ^ swz<D>(n)) * 8));
      s = mfma_32x32x16(a, qb[ks], s);
    }
    // element i holds key 8*(i/4) + 4*h + i%4 of the tile; mask keys >= lim
    const int lim = vcount - t * C::TK - 4 * h;
    if (lim < C::TK - 4) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) >= lim) s[i] = -kInf;
    }
    float mx = -kInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, partner32(mx)) * cl;
    const float m_new = (mx > m_run + kSlack) ? mx : m_run;
    const float m_ref = (m_new == -kInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    m_run = m_new;
    float ls = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = fast_exp2(fmaf(s[i], cl, -m_ref));
      ls += pv;
      pb[i >> 3][i & 7] = (__bf16)pv;
    }
    l_run = fmaf(l_run, alpha, ls);
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] *= alpha;
    }
    // O^T += V^T P^T; A operand slot j of lane (d = l%32, half h) is key
    // 16*ks2 + 8*(j/4) + 4*h + j%4 (the key of slot j of this lane's P^T)
    const int vr = 4 * h + ((l & 15) >> 2);
    const int vd = 16 * ((l >> 4) & 1) + 4 * (l & 3);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int d = b * 32 + vd;
      const int cch = d >> 3, within = d & 7;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const int r0 = 16 * ks2 + vr, r1 = r0 + 8;
        const bf16x4 lo = lds_read_tr(Vs + r0 * D + ((cch ^ swz<D>(r0)) * 8) + within);
        const bf16x4 hi = lds_read_tr(Vs + r1 * D + ((cch ^ swz<D>(r1)) * 8) + within);
        acc[b] = mfma_32x32x16(cat(lo, hi), pb[ks2], acc[b]);
      }
    }
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

  const float lt = l_run + partner32(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qv) {
    const size_t row = ((size_t)bh * p.Nq + qrow) * D;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = b * 32 + 8 * q4 + 4 * h;
        f32x4 v = {acc[b][4 * q4] * inv, acc[b][4 * q4 + 1] * inv, acc[b][4 * q4 + 2] * inv,
                   acc[b][4 * q4 + 3] * inv};
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

template <int D, int G, int S>
void launch_ring(const Params& p, dim3 grid, int k, hipStream_t st) {
  using C = Cfg<D, G, S>;
  const size_t lds = (size_t)k * 4;
  static const bool attr = allow_dynamic_lds((const void*)sparse_ring_kernel<D, G, S>, 160 * 1024 - 1024);
  (void)attr;
  hipLaunchKernelGGL((sparse_ring_kernel<D, G, S>), grid, dim3(C::NT), lds, st, p);
}

}  // namespace

constexpr int kRingStages = 2;

// Largest selection that fits the ring and the index list in one workgroup's LDS.
int sparse_max_k(int d) { return (160 * 1024 - 1024 - kRingStages * 2 * 32 * d * 2) / 4; }

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
  if (s.d == 128 && s.G == 64) launch_ring<128, 64, kRingStages>(p, grid, s.k, st);
  else if (s.d == 128) launch_ring<128, 128, kRingStages>(p, grid, s.k, st);
  else if (s.G == 64) launch_ring<64, 64, kRingStages>(p, grid, s.k, st);
  else launch_ring<64, 128, kRingStages>(p, grid, s.k, st);
  return hipGetLastError();
}

}  // namespace mcs
