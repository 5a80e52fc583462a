// Gathered sparse attention with the residual (reuse step and anchor
// epilogue) for bf16 inputs on gfx950.
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
// The copy offsets come from the group's index list through a ring of eight
// tiles' offsets in LDS, refilled from global memory a tile pair at a time
// (loaded in one half-iteration, stored in the next, read two pairs later),
// so the LDS a workgroup needs does not grow with k: four K/V slots plus one
// slot for the ring and the query-row table, 40 KB at d = 128, which keeps
// four workgroups on a CU.
//
// Residual: R is float32 by default (bf16 on request).  The slots are no
// longer needed for K/V once the last tile pair has started, so during that
// pair the group's first residual rows are copied into them (float32: k0 in
// the first half, k1, v0 and the ring slot in the second, 16 rows each; bf16:
// k0 and k1, 32 rows each) and the epilogue reads them from LDS instead of
// waiting for HBM.  Rows beyond those 64 (G = 128) are read directly.  At the
// anchor, R is formed from the float32 dense output in the workspace.
#include <type_traits>

#include "mcs_kernels.hpp"
#include "ring.hpp"

namespace mcs {
namespace {

template <int D, int G>
struct SparseCfg {
  static constexpr int NW = G / 32;
  static constexpr int NT = 64 * NW;
  static constexpr int TK = 32;                          // keys per tile
  static constexpr int CH = D / 8;                       // 16-byte chunks per bf16 row
  static constexpr int ROWS_PER_LOAD = 64 / CH;          // rows filled by one wave-wide load
  static constexpr int LOADS_PER_TENSOR = TK / ROWS_PER_LOAD;
  static constexpr int LOADS_PER_WAVE = LOADS_PER_TENSOR / NW;  // per tensor
  static constexpr int TENSOR_BYTES = TK * D * 2;
  static constexpr int RING_TILES = 8;                   // tiles of copy offsets held in LDS
  static constexpr int RING = RING_TILES * TK;
  // float32 residual rows: 16-byte chunks per row, rows per wave-wide load, rows per slot
  static constexpr int CHF = D / 4;
  static constexpr int FROWS_PER_LOAD = 64 / CHF;
  static constexpr int FROWS_PER_SLOT = TENSOR_BYTES / (4 * D);
  static_assert(LOADS_PER_WAVE >= 1 && LOADS_PER_TENSOR % NW == 0, "load split");
  static_assert(FROWS_PER_SLOT == 16, "float32 residual rows per slot");
  static_assert(RING * 4 + G * 4 + NW * 4 <= TENSOR_BYTES, "ring slot tables");
};

struct Params {
  const __bf16 *Q, *K, *V;
  const int32_t *perm, *idx;
  const float* Ofull;  // anchor: float32 dense output [BH, Nq, D]
  void* R;             // anchor: written; reuse: read (may be null); float32 or bf16
  __bf16* O;
  int Nq, Nkv, k, c, n_units, per_xcd;
  float c_log2;
  int causal_block, q_offset;
  int anchor;
};

// 16-byte chunk c of float32 residual row r (of a slot) sits at chunk c ^ fswz(r).
__device__ __forceinline__ int fswz(int r) { return r & 15; }

template <int D, int G, bool RF32>
__global__ __launch_bounds__(2 * G) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_ring_kernel(Params p) {
  using C = SparseCfg<D, G>;
  using RT = typename std::conditional<RF32, float, __bf16>::type;
  __shared__ __attribute__((aligned(1024))) unsigned char k0[C::TENSOR_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[C::TENSOR_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[C::TENSOR_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[C::TENSOR_BYTES];
  // offset ring, query rows and per-wave key counts; float32 residual rows at the end
  __shared__ __attribute__((aligned(1024))) unsigned char xs[C::TENSOR_BYTES];
  int* const s_ring = (int*)xs;
  int* const s_qrow = s_ring + C::RING;
  int* const s_kmax = s_qrow + G;

  const int unit = xcd_unit(blockIdx.x, p.per_xcd);
  if (unit >= p.n_units) return;
  const int bh = unit / p.c, g = unit - bh * p.c;
  const int w = wave_id(), l = lane_id(), n = l & 31;
  const int klast = p.Nkv - 1, kl = p.k - 1;
  // caller data is not validated on the device; clamping keeps every access in bounds
  const int32_t* gidx = p.idx + ((size_t)bh * p.c + g) * p.k;
  // byte offset of selected row i (positions past the list repeat its last row)
  auto row_off = [&](int i) { return min(max(gidx[min(i, kl)], 0), klast) * (2 * D); };
  // the ring holds the offsets of tiles 0..5 to begin with
  for (int i = threadIdx.x; i < 6 * C::TK; i += C::NT) s_ring[i] = row_off(i);
  const int gsize = min(G, p.Nq - g * G);
  const int qloc = w * 32 + n;
  const bool qv = qloc < gsize;
  const int32_t* gperm = p.perm + (size_t)bh * p.Nq + (size_t)g * G;
  const int qrow = min(max(gperm[qv ? qloc : 0], 0), p.Nq - 1);
  if (l < 32) s_qrow[qloc] = qrow;  // rows of the residual copies (a valid row for every slot)

  // number of selected keys visible to this lane's query (a prefix: ascending list)
  int vcount = qv ? p.k : 0;
  if (p.causal_block) {
    // lower bound of the query's visibility limit in the list, in LDS (k0 as
    // scratch before the first copy) when the list fits, else in global memory
    constexpr int kScratch = C::TENSOR_BYTES / 4;
    int* scr = (int*)k0;
    const bool lds = p.k <= kScratch;
    if (lds)
      for (int i = threadIdx.x; i < p.k; i += C::NT) scr[i] = gidx[i];
    __syncthreads();
    if (qv) {
      const long long lim64 = ((long long)(p.q_offset + qrow) / p.causal_block + 1) * p.causal_block;
      const int lim = lim64 < p.Nkv ? (int)lim64 : p.Nkv;
      int lo = 0, hi = p.k;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((lds ? scr[mid] : gidx[mid]) < lim) lo = mid + 1; else hi = mid;
      }
      vcount = lo;
    }
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
      o[j] = s_ring[(t % C::RING_TILES) * C::TK + r] | ((lchunk ^ swz<D>(r)) * 16);
    }
  };
  auto issue = [&](__amdgpu_buffer_rsrc_t res, const int (&o)[C::LOADS_PER_WAVE], unsigned char* slot) {
#pragma unroll
    for (int j = 0; j < C::LOADS_PER_WAVE; ++j) dma16_buf(res, o[j], slot + (wu + C::NW * j) * 1024);
  };
  // ring refill: the offsets of tiles t+6 and t+7, loaded in the first half
  // of pair t and stored in the second (their ring entries held tiles t-2 and
  // t-1, read two pairs earlier); threads 0 .. 2*TK-1 carry one entry each
  int refill = 0;
  const bool rthr = threadIdx.x < 2 * C::TK;
  // residual rows of the group go through LDS: float32 16 per slot, bf16 32 per slot
  const bool rcopy = !p.anchor && p.R != nullptr;
  const RT* Rh = rcopy ? (const RT*)p.R + (size_t)bh * p.Nq * D : nullptr;
  constexpr int RPS = RF32 ? C::FROWS_PER_SLOT : C::TK;  // residual rows per slot
  constexpr int RROWS = G < 4 * RPS ? G : (RF32 ? 4 * RPS : 2 * RPS);
  // copies of residual rows [RPS*part, RPS*part + RPS) into a slot, laid out
  // like a K tile (bf16) or as float32 rows with chunks swizzled by fswz;
  // rows[j]: the token row this lane copies in its j-th wave-wide load
  auto r_rows = [&](int part, int (&rows)[C::LOADS_PER_WAVE]) {
#pragma unroll
    for (int j = 0; j < C::LOADS_PER_WAVE; ++j) {
      const int r = (RF32 ? C::FROWS_PER_LOAD * (wu + C::NW * j) + l / C::CHF
                          : C::ROWS_PER_LOAD * (wu + C::NW * j) + lrow0);
      rows[j] = s_qrow[min(part * RPS + r, G - 1)];
    }
  };
  auto issue_r = [&](const int (&rows)[C::LOADS_PER_WAVE], unsigned char* slot) {
#pragma unroll
    for (int j = 0; j < C::LOADS_PER_WAVE; ++j) {
      if constexpr (RF32) {
        const int r = C::FROWS_PER_LOAD * (wu + C::NW * j) + l / C::CHF;
        dma16(Rh + (size_t)rows[j] * D + ((l % C::CHF) ^ fswz(r)) * 4, slot + (wu + C::NW * j) * 1024);
      } else {
        const int r = C::ROWS_PER_LOAD * (wu + C::NW * j) + lrow0;
        dma16(Rh + (size_t)rows[j] * D + (lchunk ^ swz<D>(r)) * 8, slot + (wu + C::NW * j) * 1024);
      }
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
    if (!last) {
      offsets(t + 2, ok);
      issue(kres, ok, k0);
      if (rthr) refill = row_off((t + 6) * C::TK + (int)threadIdx.x);
    } else if (rcopy) {
      int rows[C::LOADS_PER_WAVE];
      r_rows(0, rows);
      issue_r(rows, k0);  // k0 is free from here on
    }
    issue(vres, ov, v1);
    st.template step<1, 0>(sa, v0, vcount - t * C::TK, p.c_log2, k1, sb);
    // K(t+2) in k0, V(t+1) in v1, scores of tile t+1 in sb; ok = offsets of tile t+2
    wait_vmcnt<0>();
    __syncthreads();
    if (!last) {
      if (rthr) s_ring[((t + 6) % C::RING_TILES) * C::TK + threadIdx.x] = refill;
      offsets(t + 3, ov);
      issue(kres, ov, k1);
      issue(vres, ok, v0);
    } else if (rcopy && RROWS > RPS) {
      // k1 and v0 are free from here on, and (float32) the ring slot once every
      // wave has read its rows from the query-row table it holds
      int rows1[C::LOADS_PER_WAVE], rows2[C::LOADS_PER_WAVE], rows3[C::LOADS_PER_WAVE];
      r_rows(1, rows1);
      if constexpr (RF32) {
        r_rows(2, rows2);
        r_rows(3, rows3);
        __syncthreads();
        issue_r(rows2, v0);
        issue_r(rows3, xs);
      }
      issue_r(rows1, k1);
    }
    // on the last pair the scores formed here (from k0) belong to no tile and are never used
    st.template step<1, 0>(sb, v1, vcount - (t + 1) * C::TK, p.c_log2, k0, sa);
  }
  const bool rlds = rcopy && ntiles > 0;  // residual rows [0, RROWS) are in LDS
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
  // 16-byte bf16 chunk 4b+q4 of the row (float32 chunk 8b + 2q4 + h)
  auto write_out = [&](auto residual) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = b * 32 + 8 * q4 + 4 * h;
        f32x4 v = st.out4(b, q4, inv) + residual(b, q4, d0);
        const bf16x4 o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *(bf16x4*)(p.O + row + d0) = o;
      }
  };
  auto widen = [](bf16x4 r) { return f32x4{(float)r[0], (float)r[1], (float)r[2], (float)r[3]}; };
  if (p.anchor) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = b * 32 + 8 * q4 + 4 * h;
        const f32x4 r = *(const f32x4*)(p.Ofull + row + d0) - st.out4(b, q4, inv);
        if constexpr (RF32) {
          *(f32x4*)((float*)p.R + row + d0) = r;
        } else {
          const bf16x4 rb = {(__bf16)r[0], (__bf16)r[1], (__bf16)r[2], (__bf16)r[3]};
          *(bf16x4*)((__bf16*)p.R + row + d0) = rb;
        }
      }
  } else if (!p.R) {
    write_out([&](int, int, int) { return f32x4{}; });
  } else if (rlds && wu * 32 < RROWS) {
    if constexpr (RF32) {
      // row qloc sits in slot qloc / 16 (k0, k1, v0, xs), row qloc % 16
      const int s = qloc >> 4, r = qloc & 15;
      const unsigned char* slot = s == 0 ? k0 : s == 1 ? k1 : s == 2 ? v0 : xs;
      const unsigned char* rrow = slot + r * (4 * D);
      write_out([&](int b, int q4, int) { return *(const f32x4*)(rrow + 16 * ((8 * b + 2 * q4 + h) ^ fswz(r))); });
    } else {
      // this wave's residual rows sit in k0 (wave 0) or k1 (wave 1), row n, K-tile layout
      const unsigned char* rrow = (wu == 0 ? k0 : k1) + n * (2 * D) + 8 * h;
      write_out([&](int b, int q4, int) { return widen(*(const bf16x4*)(rrow + 16 * ((4 * b + q4) ^ swz<D>(n)))); });
    }
  } else {
    if constexpr (RF32)
      write_out([&](int, int, int d0) { return *(const f32x4*)((const float*)p.R + row + d0); });
    else
      write_out([&](int, int, int d0) { return widen(*(const bf16x4*)((const __bf16*)p.R + row + d0)); });
  }
}

template <int D, int G>
void launch_ring(const Params& p, dim3 grid, bool rf32, hipStream_t st) {
  if (rf32) hipLaunchKernelGGL((sparse_ring_kernel<D, G, true>), grid, dim3(SparseCfg<D, G>::NT), 0, st, p);
  else hipLaunchKernelGGL((sparse_ring_kernel<D, G, false>), grid, dim3(SparseCfg<D, G>::NT), 0, st, p);
}

}  // namespace

hipError_t launch_sparse_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                              const int32_t* perm, const int32_t* idx, const float* Ofull, void* R, bool r_f32,
                              void* O, bool anchor, hipStream_t st) {
  Params p;
  p.Q = (const __bf16*)Q; p.K = (const __bf16*)K; p.V = (const __bf16*)V;
  p.perm = perm; p.idx = idx; p.Ofull = Ofull; p.R = R; p.O = (__bf16*)O;
  p.Nq = s.Nq; p.Nkv = s.Nkv; p.k = s.k; p.c = s.c;
  p.c_log2 = s.scale * kLog2e; p.causal_block = s.causal_block; p.q_offset = s.q_offset;
  p.anchor = anchor ? 1 : 0;
  p.n_units = s.BH * s.c;
  p.per_xcd = (p.n_units + 7) / 8;
  const dim3 grid(8 * p.per_xcd);
  if (s.d == 128 && s.G == 64) launch_ring<128, 64>(p, grid, r_f32, st);
  else if (s.d == 128) launch_ring<128, 128>(p, grid, r_f32, st);
  else if (s.G == 64) launch_ring<64, 64>(p, grid, r_f32, st);
  else launch_ring<64, 128>(p, grid, r_f32, st);
  return hipGetLastError();
}

}  // namespace mcs
