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
// direct-to-LDS loads.  K and V have separate two-slot rings and each wave
// runs a software pipeline: in iteration t the scores of tile t+1 (MFMA) are
// formed next to the softmax of tile t (VALU), then O^T += V^T P^T for tile
// t.  At the start of iteration t, after one barrier, K(t+2) goes into the
// slot K(t) left and V(t+1) into the slot V(t-1) left; each copy is issued a
// full iteration before it is read.  The slots are distinct LDS objects and
// the loop is unrolled by two, so the compiler can tell the slots being read
// from the slots being filled and adds no wait for the copies in flight.
//
// Residual (reuse step): R has the input dtype.  The K slots are no longer
// needed once the last tile pair has started, so the group's first 2*TK
// residual rows are copied into them during that pair (one slot per half);
// the epilogue then reads them from LDS instead of waiting for HBM.  Rows
// beyond 2*TK (G = 128) are read directly.  At the anchor, R is formed from
// the float32 dense output in the workspace.
#include "mcs_kernels.hpp"
#include "ring.hpp"

namespace mcs {
namespace {

// Entries of the per-group offset table: k rounded up to a whole number of
// 64-key tile pairs, plus one more pair (the loop reads the offsets of up to
// two tiles past the last).
__host__ __device__ constexpr int pad_keys(int k) { return (k + 63) / 64 * 64 + 64; }

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
  static_assert(LOADS_PER_WAVE >= 1 && LOADS_PER_TENSOR % NW == 0, "load split");
};

struct Params {
  const __bf16 *Q, *K, *V;
  const int32_t *perm, *idx;
  const float* Ofull;  // anchor: float32 dense output [BH, Nq, D]
  __bf16* R;           // anchor: written; reuse: read (may be null)
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
  __shared__ __attribute__((aligned(1024))) unsigned char k0[C::TENSOR_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[C::TENSOR_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[C::TENSOR_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[C::TENSOR_BYTES];
  extern __shared__ __attribute__((aligned(16))) int s_off[];
  __shared__ int s_kmax[C::NW];
  __shared__ int s_qrow[G];

  const int unit = xcd_unit(blockIdx.x, p.per_xcd);
  if (unit >= p.n_units) return;
  const int bh = unit / p.c, g = unit - bh * p.c;
  const int w = wave_id(), l = lane_id(), n = l & 31;
  const int klast = p.Nkv - 1;
  {
    // byte offsets of the selected rows, padded with the last one so that the
    // copies of every tile (and of the two tiles past the end) read in bounds
    const int32_t* gidx = p.idx + ((size_t)bh * p.c + g) * p.k;
    const int kpad = pad_keys(p.k);
    for (int i = threadIdx.x; i < kpad; i += C::NT) s_off[i] = min(max(gidx[min(i, p.k - 1)], 0), klast) * (2 * D);
  }
  const int gsize = min(G, p.Nq - g * G);
  const int qloc = w * 32 + n;
  const bool qv = qloc < gsize;
  const int32_t* gperm = p.perm + (size_t)bh * p.Nq + (size_t)g * G;
  // caller data is not validated on the device; clamping keeps every access in bounds
  const int qrow = min(max(gperm[qv ? qloc : 0], 0), p.Nq - 1);
  if (l < 32) s_qrow[qloc] = qrow;  // rows of the residual copies (a valid row for every slot)
  __syncthreads();

  // number of selected keys visible to this lane's query (a prefix: ascending list)
  int vcount = qv ? p.k : 0;
  if (qv && p.causal_block) {
    const long long lim64 = ((long long)(p.q_offset + qrow) / p.causal_block + 1) * p.causal_block;
    const int lim = lim64 < p.Nkv ? (int)lim64 : p.Nkv;
    const int lim_off = lim * (2 * D);
    int lo = 0, hi = p.k;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] < lim_off) lo = mid + 1; else hi = mid;
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
  // rounded up to even: the loop below handles tiles in pairs with a single
  // exit (a mid-loop exit makes the compiler copy the O accumulators between
  // register sets every tile); a tile past kmax is fully masked for every
  // lane, so its maximum is -inf, the reference stays, alpha = 1 and every
  // probability is 0: it changes nothing
  const int ntiles = ((kmax + C::TK - 1) / C::TK + 1) & ~1;

  const __bf16* Kh = p.K + (size_t)bh * p.Nkv * D;
  const __bf16* Vh = p.V + (size_t)bh * p.Nkv * D;
  // this lane's part of every tile load: row r = ROWS_PER_LOAD*(wu + NW*j) + l/CH, chunk l%CH,
  // as a 32-bit byte offset into the head's K or V (a head holds < 2^31 bytes); the K copy
  // of a tile and its V copy one iteration later use the same offsets
  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform: LDS targets in scalar registers
  const int lrow0 = l / C::CH, lchunk = l % C::CH;
  const __amdgpu_buffer_rsrc_t kres = buffer_rsrc(Kh, p.Nkv * D * 2), vres = buffer_rsrc(Vh, p.Nkv * D * 2);
  auto offsets = [&](int t, int (&o)[C::LOADS_PER_WAVE]) {
#pragma unroll
    for (int j = 0; j < C::LOADS_PER_WAVE; ++j) {
      const int r = C::ROWS_PER_LOAD * (wu + C::NW * j) + lrow0;
      o[j] = s_off[t * C::TK + r] | ((lchunk ^ swz<D>(r)) * 16);
    }
  };
  auto issue = [&](__amdgpu_buffer_rsrc_t res, const int (&o)[C::LOADS_PER_WAVE], unsigned char* slot) {
#pragma unroll
    for (int j = 0; j < C::LOADS_PER_WAVE; ++j) dma16_buf(res, o[j], slot + (wu + C::NW * j) * 1024);
  };
  // residual rows [TK*part, TK*part + TK) of the group into a K slot, laid out like a K tile
  constexpr int RROWS = G < 2 * C::TK ? G : 2 * C::TK;  // rows that go through LDS
  const bool rcopy = !p.anchor && p.R != nullptr;
  const __bf16* Rh = rcopy ? p.R + (size_t)bh * p.Nq * D : nullptr;
  auto issue_r = [&](int part, unsigned char* slot) {
#pragma unroll
    for (int j = 0; j < C::LOADS_PER_WAVE; ++j) {
      const int r = C::ROWS_PER_LOAD * (wu + C::NW * j) + lrow0;
      const int row = s_qrow[min(part * C::TK + r, G - 1)];
      dma16(Rh + (size_t)row * D + (lchunk ^ swz<D>(r)) * 8, slot + (wu + C::NW * j) * 1024);
    }
  };
  f32x16 sa[1], sb[1];
  int ok[C::LOADS_PER_WAVE], ov[C::LOADS_PER_WAVE];  // offsets of the next K copy / of the next V copy
  if (ntiles > 0) {
    offsets(0, ov);
    issue(kres, ov, k0);
    issue(vres, ov, v0);
    offsets(1, ov);
    issue(kres, ov, k1);
    wait_vmcnt<0>();
    __syncthreads();
    st.template scores<1, 0>(k0, sa);
  }
  for (int t = 0; t < ntiles; t += 2) {
    const bool last = t + 2 >= ntiles;
    // K(t+1) in k1, V(t) in v0, scores of tile t in sa; ov = offsets of tile t+1
    wait_vmcnt<0>();
    __syncthreads();
    offsets(t + 2, ok);
    if (!last) issue(kres, ok, k0);
    else if (rcopy) issue_r(0, k0);  // k0 is free from here on
    issue(vres, ov, v1);
    st.template step<1, 0>(sa, v0, vcount - t * C::TK, p.c_log2, k1, sb);
    // K(t+2) in k0, V(t+1) in v1, scores of tile t+1 in sb; ok = offsets of tile t+2
    wait_vmcnt<0>();
    __syncthreads();
    offsets(t + 3, ov);
    if (!last) {
      issue(kres, ov, k1);
      issue(vres, ok, v0);
    } else if (rcopy && RROWS > C::TK) {
      issue_r(1, k1);  // k1 is free from here on
    }
    // on the last pair the scores formed here (from k0) belong to no tile and are never used
    st.template step<1, 0>(sb, v1, vcount - (t + 1) * C::TK, p.c_log2, k0, sa);
  }
  const bool rlds = rcopy && ntiles > 0;  // residual rows [0, RROWS) are in k0/k1
  if (rlds) {
    wait_vmcnt<0>();
    __syncthreads();
  }

  float lse;
  const float inv = st.finish(lse);
  if (!qv) return;
  const int h = l >> 5;
  const size_t row = ((size_t)bh * p.Nq + qrow) * D;
  // output channels d0..d0+3 of this lane: d0 = 32b + 8q4 + 4h, i.e. half h of
  // 16-byte chunk 4b+q4 of the row
  auto write_out = [&](auto residual) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = b * 32 + 8 * q4 + 4 * h;
        f32x4 v = st.out4(b, q4, inv);
        const bf16x4 rb = residual(4 * b + q4, d0);
        v[0] += (float)rb[0];
        v[1] += (float)rb[1];
        v[2] += (float)rb[2];
        v[3] += (float)rb[3];
        const bf16x4 o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *(bf16x4*)(p.O + row + d0) = o;
      }
  };
  if (p.anchor) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = b * 32 + 8 * q4 + 4 * h;
        const f32x4 r = *(const f32x4*)(p.Ofull + row + d0) - st.out4(b, q4, inv);
        const bf16x4 rb = {(__bf16)r[0], (__bf16)r[1], (__bf16)r[2], (__bf16)r[3]};
        *(bf16x4*)(p.R + row + d0) = rb;
      }
  } else if (!p.R) {
    write_out([&](int, int) { return bf16x4{}; });
  } else if (rlds && wu * 32 < RROWS) {
    // this wave's residual rows sit in k0 (wave 0) or k1 (wave 1), row n, K-tile layout
    const unsigned char* rrow = (wu == 0 ? k0 : k1) + n * (2 * D) + 8 * h;
    write_out([&](int chunk, int) { return *(const bf16x4*)(rrow + 16 * (chunk ^ swz<D>(n))); });
  } else {
    write_out([&](int, int d0) { return *(const bf16x4*)(p.R + row + d0); });
  }
}

template <int D, int G>
void launch_ring(const Params& p, dim3 grid, int k, hipStream_t st) {
  using C = SparseCfg<D, G>;
  const size_t lds = (size_t)pad_keys(k) * 4;
  static const bool attr = allow_dynamic_lds((const void*)sparse_ring_kernel<D, G>,
                                             160 * 1024 - 4 * C::TENSOR_BYTES - 1024);
  (void)attr;
  hipLaunchKernelGGL((sparse_ring_kernel<D, G>), grid, dim3(C::NT), lds, st, p);
}

}  // namespace

hipError_t launch_sparse_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                              const int32_t* perm, const int32_t* idx, const float* Ofull, void* R, void* O,
                              bool anchor, hipStream_t st) {
  Params p;
  p.Q = (const __bf16*)Q; p.K = (const __bf16*)K; p.V = (const __bf16*)V;
  p.perm = perm; p.idx = idx; p.Ofull = Ofull; p.R = (__bf16*)R; p.O = (__bf16*)O;
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
