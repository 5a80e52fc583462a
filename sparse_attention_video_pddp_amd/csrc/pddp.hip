// Fast-PDDP query grouping (MC-Sparse review, blog.secrett2633.cloud,
// section 3: similar queries are packed into equal-size, tile-aligned groups
// by Principal Direction Divisive Partitioning).
//
// The tree is processed level by level.  Groups are numbered depth-first, so
// every node is one contiguous range perm[start, start+n) of its head, and
// the node's shape (start, n, c groups) follows from its slot number alone.
// For a node with c >= 2 groups:
//   1. S = sum x and the raw scatter sum x x^T over the node's rows: bf16
//      rows through v_mfma_f32_32x32x16_bf16 (exact products, fp32 sums over
//      64-row tiles, fp64 across tiles), fp32 rows with fp64 FMAs;
//   2. C = sum x x^T - S S^T / n (fp64) and the fixed-step power iteration
//      v <- C v / ||C v|| from v0 = 1/sqrt(d) in fp64 (a zero product keeps v);
//   3. projections p_i = x_i . v - (S/n) . v in fp64, keyed by float(p_i);
//   4. the floor(c/2)*G members of smallest key, equal keys lowest position
//      first, go left, the rest right, both in their previous order (members
//      stay in ascending token order, so position order is index order).
//
// Two schedules.  Levels whose nodes are larger than `cr` rows (the top of
// the tree, few nodes) are spread over many workgroups: row chunks of cr
// rows produce partial sums (step 1), an ordered reduction adds them, one
// workgroup per node iterates (step 2), row chunks project (step 3) and one
// workgroup per node splits (step 4, select.hpp).  Smaller nodes are done by
// one workgroup each from start to end, with the projection keys and member
// ids kept in registers.
//
// In step 1 the gathered rows of a 64-row tile are copied straight into LDS
// (global_load_lds, 16 bytes per lane) in a two-slot ring, row-major with the
// 16-byte chunks XOR-swizzled per row; both MFMA operands (x^T blocks) are
// read with ds_read_b64_tr_b16.  Wave w holds column block w of the scatter
// matrix in the MFMA output layout (lane: one column, 16 rows per 32-row
// block), so C v needs only an in-lane sum and one half-wave exchange.
#include <algorithm>
#include <type_traits>

#include "mcs_kernels.hpp"
#include "ring.hpp"
#include "select.hpp"

namespace mcs {
namespace {

constexpr int kNodeThreads = 256;
constexpr int kSplitThreads = 512;
constexpr int kSplitWideThreads = 1024;  // nodes of 32769..81920 rows: 80 keys per thread
constexpr int kProjRows = 512;      // rows per workgroup of the projection kernel
constexpr int kMaxChunkRows = 4096;  // row chunk of the many-workgroup levels; larger nodes split there

struct PddpParams {
  const void* Q;
  int32_t* perm;
  int32_t* tmp;
  uint32_t* keys;
  double* part;  // [BH][nslots][pmax][D + D*D] partial (S, sum x x^T) per row chunk
  double* red;   // [BH][nslots][D + D*D] their sums
  double* vec;   // [BH][nslots][D + 1] direction v and (S/n) . v
  int Nq, G, iters, level, cr, pmax;
  int pj_pmax;  // projection chunks (of kProjRows rows) per node at this level
};

struct Node {
  int start, n, c;
};

// Shape of node `slot` of `level` (c == 0: the slot lies under a leaf).
__device__ __forceinline__ Node pddp_node(int slot, int level, int Nq, int G) {
  Node nd{0, Nq, (Nq + G - 1) / G};
  for (int b = level - 1; b >= 0; --b) {
    if (nd.c <= 1) return Node{0, 0, 0};
    const int cL = nd.c >> 1, nL = cL * G;
    if ((slot >> b) & 1) {
      nd.start += nL;
      nd.n -= nL;
      nd.c -= cL;
    } else {
      nd.n = nL;
      nd.c = cL;
    }
  }
  return nd;
}

template <int D>
struct GramCfg {
  static constexpr int NB = D / 32;
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int RPL = 64 / CH;       // rows per wave-wide copy
  static constexpr int LPW = 64 / RPL / 4;  // wave-wide copies per wave per 64-row tile
  static constexpr int TILE_BYTES = 64 * D * 2;
  static constexpr int FS = D + 4;          // fp32 staging row stride
};

template <int D, bool BF16>
struct GramLds {
  static constexpr int SLOT0 = BF16 ? GramCfg<D>::TILE_BYTES : 64 * GramCfg<D>::FS * 4;
  static constexpr int SLOT1 = BF16 ? GramCfg<D>::TILE_BYTES : 16;
};

// Step 1 over member rows [r0, r1) of a node (nperm: the node's members).
// cacc (waves w < NB): sum x x^T, element (bi, i) = row 32*bi + 8*(i/4) +
// 4*h + i%4, column 32*w + lane%32.  sS[0..D): sum x.  Ends with a barrier.
template <int D, bool BF16>
__device__ void gram_rows(const void* Qv, size_t hbase, const int32_t* nperm, int r0, int r1,
                          unsigned char* slot0, unsigned char* slot1, double (&cacc)[D / 32][16], double* sS) {
  using C = GramCfg<D>;
  constexpr int NB = C::NB;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
#pragma unroll
  for (int bi = 0; bi < NB; ++bi)
#pragma unroll
    for (int i = 0; i < 16; ++i) cacc[bi][i] = 0.0;

  if constexpr (BF16) {
    const __bf16* Qh = (const __bf16*)Qv + hbase * D;
    // operand reads (transposing): lane l gets channel 32*b + l%32 of rows
    // 4h + j (first read) and 8 + 4h + j (second read), j = 0..3, of each
    // 16-row step; rows enter both operands in the same order
    const int vr = 4 * h + ((l & 15) >> 2);
    const int c0 = 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
    const int ob0 = vr * (2 * D) + 8 * (l & 1) + 16 * (c0 ^ swz<D>(vr));
    const int ob1 = (8 + vr) * (2 * D) + 8 * (l & 1) + 16 * (c0 ^ swz<D>(8 + vr));
    const int lrow0 = l / C::CH, lchunk = l % C::CH;
    const int ntiles = (r1 - r0 + 63) / 64;
    // column sums: lane (n, h) of wave w keeps element n%16 of the ones-product,
    // i.e. S[32w + 8((n%16)/4) + 4h + n%4]
    double sacc = 0.0;
    const int si = ln & 15;
    int ids[C::LPW];
    auto load_ids = [&](int t) {
#pragma unroll
      for (int j = 0; j < C::LPW; ++j) {
        const int r = C::RPL * (w + 4 * j) + lrow0;
        ids[j] = nperm[min(r0 + t * 64 + r, r1 - 1)];  // tail rows repeat the last row (masked below)
      }
    };
    auto issue = [&](unsigned char* slot) {
#pragma unroll
      for (int j = 0; j < C::LPW; ++j) {
        const int li = w + 4 * j;
        const int r = C::RPL * li + lrow0;
        dma16(Qh + (size_t)ids[j] * D + ((lchunk ^ swz<D>(r)) * 8), slot + li * 1024);
      }
    };
    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (__bf16)1.0f;
    // x^T operand of channel block b for 16-row step ks2, rows >= valid zeroed
    auto operand = [&](const unsigned char* slot, int b, int ks2, int valid) {
      const unsigned char* base = slot + 16 * (2 * D) * ks2;
      bf16x8 op = cat(lds_read_tr(base + (ob0 ^ (64 * b))), lds_read_tr(base + (ob1 ^ (64 * b))));
      if (valid < 64) {
        const __bf16 z = (__bf16)0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          op[j] = 16 * ks2 + 4 * h + j < valid ? op[j] : z;
          op[4 + j] = 16 * ks2 + 8 + 4 * h + j < valid ? op[4 + j] : z;
        }
      }
      return op;
    };
    // two fp32 accumulators live at a time (row blocks outer), which keeps the
    // kernel within 256 registers per lane
    auto compute = [&](const unsigned char* slot, int valid) {
      if (w >= NB) return;
      bf16x8 ow[4];
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2) ow[ks2] = operand(slot, w, ks2, valid);
      f32x16 accS = {};
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2) accS = mfma_32x32x16(ow[ks2], ones, accS);
#pragma unroll
      for (int bi = 0; bi < NB; bi += 2) {  // two independent accumulators
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int ks2 = 0; ks2 < 4; ++ks2) {
          acc0 = mfma_32x32x16(operand(slot, bi, ks2, valid), ow[ks2], acc0);
          acc1 = mfma_32x32x16(operand(slot, bi + 1, ks2, valid), ow[ks2], acc1);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          cacc[bi][i] += (double)acc0[i];
          cacc[bi + 1][i] += (double)acc1[i];
        }
      }
      float sv = accS[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) sv = (si == i) ? accS[i] : sv;
      sacc += (double)sv;
    };
    if (ntiles > 0) {
      load_ids(0);
      issue(slot0);
      if (ntiles > 1) load_ids(1);
    }
    for (int t = 0; t < ntiles; t += 2) {
      wait_vmcnt<0>();
      __syncthreads();
      if (t + 1 < ntiles) {
        issue(slot1);
        if (t + 2 < ntiles) load_ids(t + 2);
      }
      compute(slot0, r1 - r0 - t * 64);
      if (t + 1 >= ntiles) break;
      wait_vmcnt<0>();
      __syncthreads();
      if (t + 2 < ntiles) {
        issue(slot0);
        if (t + 3 < ntiles) load_ids(t + 3);
      }
      compute(slot1, r1 - r0 - (t + 1) * 64);
    }
    if (w < NB && ln < 16) sS[32 * w + 8 * (si >> 2) + 4 * h + (si & 3)] = sacc;
    __syncthreads();
  } else {
    const float* Qf = (const float*)Qv + hbase * D;
    float* Xs = (float*)slot0;
    double ssum = 0.0;
    for (int rr = r0; rr < r1; rr += 64) {
      const int rows = min(64, r1 - rr);
      for (int e = tid; e < 64 * (D / 4); e += blockDim.x) {
        const int r = e / (D / 4), ch = e % (D / 4);
        f32x4 v = {};
        if (r < rows) v = *(const f32x4*)(Qf + (size_t)nperm[rr + r] * D + ch * 4);
        *(f32x4*)(Xs + r * C::FS + ch * 4) = v;
      }
      __syncthreads();
      if (tid < D)
        for (int r = 0; r < 64; ++r) ssum += (double)Xs[r * C::FS + tid];
      if (w < NB) {
        for (int r = 0; r < 64; ++r) {
          const double xc = (double)Xs[r * C::FS + w * 32 + ln];
#pragma unroll
          for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              cacc[bi][i] = fma((double)Xs[r * C::FS + bi * 32 + 8 * (i >> 2) + 4 * h + (i & 3)], xc, cacc[bi][i]);
        }
      }
      __syncthreads();
    }
    if (tid < D) sS[tid] = ssum;
    __syncthreads();
  }
}

// Step 2.  cacc holds sum x x^T (layout of gram_rows), sS the column sums
// (visible to all threads).  Leaves v in sV and returns (S/n) . v.
// With v_k = y_k / ||y_k||, the iteration runs as y_{k+1} = C y_k / ||y_k||:
// the norm of y_k is reduced while y_{k+1} is formed, so one barrier per step
// suffices (y double-buffered in sY).  If C v_k = 0 the direction stays v_k.
template <int D>
__device__ double centre_and_iterate(double (&cacc)[D / 32][16], const double* sS, double* sV, double (*sY)[D],
                                     double (*sRed)[4], int n, int iters) {
  constexpr int NB = D / 32;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
  const bool gw = w < NB;
  const double inv_n = 1.0 / (double)n;
  if (gw) {
    const double sc = sS[w * 32 + ln] * inv_n;
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i) cacc[bi][i] -= sS[bi * 32 + 8 * (i >> 2) + 4 * h + (i & 3)] * sc;
  }
  // y_0 = v_0 = 1/sqrt(d) (unit norm)
  if (tid < D) sY[0][tid] = 1.0 / sqrt((double)D);
  if (tid < 4) sRed[0][tid] = tid == 0 ? 1.0 : 0.0;
  __syncthreads();
  int cur = 0;   // buffer holding y_k
  int last = 0;  // buffer of the last y with a nonzero norm
  for (int it = 0; it < iters; ++it) {
    const double nrm2 = (sRed[cur][0] + sRed[cur][1]) + (sRed[cur][2] + sRed[cur][3]);
    if (nrm2 == 0.0) break;  // C v = 0: keep the previous direction
    last = cur;
    const double inv = 1.0 / sqrt(nrm2);
    double wv = 0.0;
    if (gw) {
      double part[NB];  // independent FMA chains, one per row block
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
        part[bi] = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) part[bi] = fma(cacc[bi][i], sY[cur][bi * 32 + 8 * (i >> 2) + 4 * h + (i & 3)], part[bi]);
      }
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) wv += part[bi];
      wv += partner32_f64(wv);
      wv *= inv;
    }
    const double sq = wave_sum_f64((gw && h == 0) ? wv * wv : 0.0);
    const int nxt = cur ^ 1;
    if (gw && h == 0) sY[nxt][w * 32 + ln] = wv;
    if (l == 0 && w < 4) sRed[nxt][w] = gw ? sq : 0.0;
    __syncthreads();
    cur = nxt;
  }
  {
    const double nrm2 = (sRed[cur][0] + sRed[cur][1]) + (sRed[cur][2] + sRed[cur][3]);
    if (nrm2 != 0.0) last = cur;
  }
  const double nl = (sRed[last][0] + sRed[last][1]) + (sRed[last][2] + sRed[last][3]);
  const double inv = 1.0 / sqrt(nl);
  if (tid < D) sV[tid] = sY[last][tid] * inv;
  __syncthreads();
  const double mv = wave_sum_f64(tid < D ? sS[tid] * inv_n * sV[tid] : 0.0);
  if (l == 0 && w < 4) sRed[cur ^ 1][w] = mv;  // buffer no longer read
  __syncthreads();
  const double muv = (sRed[cur ^ 1][0] + sRed[cur ^ 1][1]) + (sRed[cur ^ 1][2] + sRed[cur ^ 1][3]);
  __syncthreads();
  return muv;
}

// Step 3: projections of whole rows by groups of D/8 lanes (8 channels per
// lane, one coalesced row read per group); the key is the flipped order key
// of float(x . v - muv), so that the left child (smallest projections) is the
// selection of largest keys.
template <int D, bool BF16>
struct RowProjector {
  static constexpr int LPR = D / 8;     // lanes per row
  static constexpr int RPW = 64 / LPR;  // rows per wave step
  double vv[8];
  int q;
  __device__ __forceinline__ void init(const double* sV) {
    q = lane_id() % LPR;
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = sV[8 * q + j];
  }
  using Raw = typename std::conditional<BF16, bf16x8, f32x4[2]>::type;
  struct Row {
    Raw x;
  };
  __device__ __forceinline__ Row load(const void* Qv, size_t row) const {
    Row r;
    if constexpr (BF16) {
      r.x = *(const bf16x8*)((const __bf16*)Qv + row * D + 8 * q);
    } else {
      const float* qp = (const float*)Qv + row * D + 8 * q;
      r.x[0] = *(const f32x4*)qp;
      r.x[1] = *(const f32x4*)(qp + 4);
    }
    return r;
  }
  // Every lane of the row's group returns the key.
  __device__ __forceinline__ uint32_t key(const Row& r, double muv) const {
    double d = 0.0;
    if constexpr (BF16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) d = fma((double)(float)r.x[j], vv[j], d);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) d = fma((double)r.x[0][j], vv[j], d);
#pragma unroll
      for (int j = 0; j < 4; ++j) d = fma((double)r.x[1][j], vv[4 + j], d);
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) d += __shfl_xor(d, o, 64);
    const float pf = (float)(d - muv) + 0.0f;  // + 0 folds -0 into +0
    return ~float_order_key(pf);
  }
};

// Keys of member rows [r0, r1) (positions within the node): f(i, key) once per row.
template <int D, bool BF16, int NT, class F>
__device__ __forceinline__ void project_rows(const void* Qv, size_t hbase, const int32_t* nperm, int r0, int r1,
                                             const double* sV, double muv, F&& f) {
  using P = RowProjector<D, BF16>;
  P pr;
  pr.init(sV);
  constexpr int U = 4;  // rows per lane group in flight
  const int w = wave_id(), sub = lane_id() / P::LPR;
  const int step = NT / 64 * P::RPW;
  for (int b = r0 + w * P::RPW; b < r1; b += U * step) {
    int id[U];
#pragma unroll
    for (int u = 0; u < U; ++u) id[u] = nperm[min(b + u * step + sub, r1 - 1)];
    typename P::Row x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = pr.load(Qv, hbase + id[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = b + u * step + sub;
      const uint32_t k = pr.key(x[u], muv);
      if (i < r1 && pr.q == 0) f(i, k);
    }
  }
}

struct NoKeys {
  __device__ __forceinline__ uint32_t operator()(int) const { return 0u; }
};

struct LdsKeys {
  const uint32_t* k;
  __device__ __forceinline__ uint32_t operator()(int j) const { return k[j]; }
};

struct GlobalKeys {
  const uint32_t* k;
  __device__ __forceinline__ uint32_t operator()(int j) const { return k[j]; }
};

// ---- one workgroup per node ------------------------------------------------
template <int D, bool BF16, int VPT>
__global__ __launch_bounds__(kNodeThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void pddp_node_kernel(PddpParams p) {
  using L = GramLds<D, BF16>;
  using Sel = BlockSelect<kNodeThreads, VPT>;
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[L::SLOT0];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[L::SLOT1];
  __shared__ double sS[D], sV[D], sY[2][D], sRed[2][4];
  __shared__ typename Sel::Shared sh;
  __shared__ uint32_t s_keys[VPT * kNodeThreads];
  const int bh = blockIdx.y;
  const Node nd = pddp_node(blockIdx.x, p.level, p.Nq, p.G);
  if (nd.c <= 1) return;
  const size_t hbase = (size_t)bh * p.Nq;
  int32_t* nperm = p.perm + hbase + nd.start;
  double cacc[D / 32][16];
  gram_rows<D, BF16>(p.Q, hbase, nperm, 0, nd.n, slot0, slot1, cacc, sS);
  const double muv = centre_and_iterate<D>(cacc, sS, sV, sY, sRed, nd.n, p.iters);
  project_rows<D, BF16, kNodeThreads>(p.Q, hbase, nperm, 0, nd.n, sV, muv, [&](int i, uint32_t k) { s_keys[i] = k; });
  __syncthreads();
  Sel sel;
  sel.n = nd.n;
  int ids[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) ids[i] = nperm[min(i * kNodeThreads + (int)threadIdx.x, nd.n - 1)];
  sel.load(LdsKeys{s_keys});
  const int nL = (nd.c >> 1) * p.G;
  uint32_t T;
  int tie_need;
  sel.threshold(NoKeys{}, nL, sh, T, tie_need);  // its barriers also retire every read of nperm
  sel.split(NoKeys{}, T, tie_need, sh, [&](int i, int, bool s, int pos) {
    const int dst = s ? pos : nL + pos;
    if (dst < nd.n) nperm[dst] = ids[i];
  });
}

// ---- small nodes ------------------------------------------------------------
// Nodes of at most kSmallRows rows (the deep levels: thousands of nodes, each a
// chain of latencies) run with a lighter state so that four workgroups share a
// CU: the scatter sums of all tiles stay in the fp32 MFMA accumulators (exact
// bf16 products, fp32 sums over at most kSmallRows rows), the centring is
// done in fp64 and the power iteration runs in fp32 (C rounded to fp32); the
// projections stay fp64.  K tiles of 32 rows in a two-slot ring of 8 KB.
constexpr int kSmallRows = 512;

template <int D>
__global__ __launch_bounds__(kNodeThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void pddp_small_kernel(PddpParams p) {
  constexpr int NB = D / 32;
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int RPL = 64 / CH;         // rows per wave-wide copy
  constexpr int TR = 32;               // rows per tile
  constexpr int LPW = TR / RPL / 4;    // wave-wide copies per wave per tile
  constexpr int TILE = TR * D * 2;
  constexpr int VPT = kSmallRows / kNodeThreads;
  static_assert(LPW >= 1, "tile copy split");
  using Sel = BlockSelect<kNodeThreads, VPT>;
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[TILE];
  __shared__ double sS[D], sV[D], sMu[4];
  __shared__ float sY[2][D], sRed[2][4];
  __shared__ typename Sel::Shared sh;
  __shared__ uint32_t s_keys[kSmallRows];
  const int bh = blockIdx.y;
  const Node nd = pddp_node(blockIdx.x, p.level, p.Nq, p.G);
  if (nd.c <= 1) return;
  const size_t hbase = (size_t)bh * p.Nq;
  int32_t* nperm = p.perm + hbase + nd.start;
  const int n = nd.n;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const bool gw = w < NB;

  // ---- 1. scatter sums, fp32 over all tiles ---------------------------------
  const __bf16* Qh = (const __bf16*)p.Q + hbase * D;
  const int vr = 4 * h + ((l & 15) >> 2);
  const int c0 = 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
  const int ob0 = vr * (2 * D) + 8 * (l & 1) + 16 * (c0 ^ swz<D>(vr));
  const int ob1 = (8 + vr) * (2 * D) + 8 * (l & 1) + 16 * (c0 ^ swz<D>(8 + vr));
  const int lrow0 = l / CH, lchunk = l % CH;
  const int ntiles = (n + TR - 1) / TR;
  int ids[LPW];
  auto load_ids = [&](int t) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) ids[j] = nperm[min(t * TR + RPL * (wu + 4 * j) + lrow0, n - 1)];
  };
  auto issue = [&](unsigned char* slot) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int r = RPL * (wu + 4 * j) + lrow0;
      dma16(Qh + (size_t)ids[j] * D + ((lchunk ^ swz<D>(r)) * 8), slot + (wu + 4 * j) * 1024);
    }
  };
  bf16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (__bf16)1.0f;
  f32x16 acc[NB], accS = {};
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
  auto compute = [&](const unsigned char* slot, int valid) {
    if (!gw) return;
#pragma unroll
    for (int ks2 = 0; ks2 < TR / 16; ++ks2) {
      const unsigned char* base = slot + 16 * (2 * D) * ks2;
      bf16x8 op[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) op[b] = cat(lds_read_tr(base + (ob0 ^ (64 * b))), lds_read_tr(base + (ob1 ^ (64 * b))));
      if (valid < TR) {
        const __bf16 z = (__bf16)0.0f;
        // rows of this lane relative to the tail, recomputed here (an opaque
        // copy keeps the compiler from hoisting the comparisons out of the
        // tile loop and spilling them)
        int rel = valid - 16 * ks2 - 4 * h;
        asm volatile("" : "+v"(rel));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool k0 = j < rel, k1 = 8 + j < rel;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            op[b][j] = k0 ? op[b][j] : z;
            op[b][4 + j] = k1 ? op[b][4 + j] : z;
          }
        }
      }
      bf16x8 ow = op[0];
#pragma unroll
      for (int b = 1; b < NB; ++b) ow = (b == w) ? op[b] : ow;
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) acc[bi] = mfma_32x32x16(op[bi], ow, acc[bi]);
      accS = mfma_32x32x16(ow, ones, accS);
    }
  };
  load_ids(0);
  issue(slot0);
  if (ntiles > 1) load_ids(1);
  for (int t = 0; t < ntiles; t += 2) {
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 1 < ntiles) {
      issue(slot1);
      if (t + 2 < ntiles) load_ids(t + 2);
    }
    compute(slot0, n - t * TR);
    if (t + 1 >= ntiles) break;
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 2 < ntiles) {
      issue(slot0);
      if (t + 3 < ntiles) load_ids(t + 3);
    }
    compute(slot1, n - (t + 1) * TR);
  }
  // column sums: lane (n, h) of wave w keeps element n%16: S[32w + 8((n%16)/4) + 4h + n%4]
  {
    const int si = ln & 15;
    float sv = accS[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) sv = (si == i) ? accS[i] : sv;
    if (gw && ln < 16) sS[32 * w + 8 * (si >> 2) + 4 * h + (si & 3)] = (double)sv;
  }
  __syncthreads();

  // ---- 2. centre in fp64, iterate in fp32 ------------------------------------
  const double inv_n = 1.0 / (double)n;
  float cf[NB][16];
  if (gw) {
    const double sc = sS[w * 32 + ln] * inv_n;
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        cf[bi][i] = (float)((double)acc[bi][i] - sS[bi * 32 + 8 * (i >> 2) + 4 * h + (i & 3)] * sc);
  }
  if (tid < D) sY[0][tid] = 1.0f / sqrtf((float)D);
  if (tid < 4) sRed[0][tid] = tid == 0 ? 1.0f : 0.0f;
  __syncthreads();
  int cur = 0, last = 0;
  for (int it = 0; it < p.iters; ++it) {
    const float nrm2 = (sRed[cur][0] + sRed[cur][1]) + (sRed[cur][2] + sRed[cur][3]);
    if (nrm2 == 0.0f) break;  // C v = 0: keep the previous direction
    last = cur;
    const float inv = 1.0f / sqrtf(nrm2);
    float wv = 0.0f;
    if (gw) {
      float part[NB];
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
        part[bi] = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) part[bi] = fmaf(cf[bi][i], sY[cur][bi * 32 + 8 * (i >> 2) + 4 * h + (i & 3)], part[bi]);
      }
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) wv += part[bi];
      wv = half_sum(wv) * inv;
    }
    const float sq = wave_sum_f32((gw && h == 0) ? wv * wv : 0.0f);
    const int nxt = cur ^ 1;
    if (gw && h == 0) sY[nxt][w * 32 + ln] = wv;
    if (l == 0 && w < 4) sRed[nxt][w] = gw ? sq : 0.0f;
    __syncthreads();
    cur = nxt;
  }
  {
    const float nrm2 = (sRed[cur][0] + sRed[cur][1]) + (sRed[cur][2] + sRed[cur][3]);
    if (nrm2 != 0.0f) last = cur;
  }
  const float nl = (sRed[last][0] + sRed[last][1]) + (sRed[last][2] + sRed[last][3]);
  const double vinv = 1.0 / sqrt((double)nl);
  if (tid < D) sV[tid] = (double)sY[last][tid] * vinv;
  __syncthreads();
  const double mv = wave_sum_f64(tid < D ? sS[tid] * inv_n * sV[tid] : 0.0);
  if (l == 0 && w < 4) sMu[w] = mv;
  __syncthreads();
  const double muv = (sMu[0] + sMu[1]) + (sMu[2] + sMu[3]);

  // ---- 3, 4. projections and split -------------------------------------------
  project_rows<D, true, kNodeThreads>(p.Q, hbase, nperm, 0, n, sV, muv, [&](int i, uint32_t k) { s_keys[i] = k; });
  __syncthreads();
  Sel sel;
  sel.n = n;
  int mid[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) mid[i] = nperm[min(i * kNodeThreads + tid, n - 1)];
  sel.load(LdsKeys{s_keys});
  const int nL = (nd.c >> 1) * p.G;
  uint32_t T;
  int tie_need;
  sel.threshold(NoKeys{}, nL, sh, T, tie_need);  // its barriers also retire every read of nperm
  sel.split(NoKeys{}, T, tie_need, sh, [&](int i, int, bool s, int pos) {
    const int dst = s ? pos : nL + pos;
    if (dst < n) nperm[dst] = mid[i];
  });
}

// ---- many workgroups per node ---------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kNodeThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void pddp_gram_kernel(PddpParams p) {
  using L = GramLds<D, BF16>;
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[L::SLOT0];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[L::SLOT1];
  __shared__ double sS[D];
  const int bh = blockIdx.y, slot = blockIdx.x / p.pmax, chunk = blockIdx.x % p.pmax;
  const Node nd = pddp_node(slot, p.level, p.Nq, p.G);
  if (nd.c <= 1) return;
  const int r0 = chunk * p.cr;
  if (r0 >= nd.n) return;
  const int r1 = min(nd.n, r0 + p.cr);
  const size_t hbase = (size_t)bh * p.Nq;
  double cacc[D / 32][16];
  gram_rows<D, BF16>(p.Q, hbase, p.perm + hbase + nd.start, r0, r1, slot0, slot1, cacc, sS);
  const int nslots = 1 << p.level;
  double* out = p.part + (((size_t)bh * nslots + slot) * p.pmax + chunk) * (D + D * D);
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
  if (tid < D) out[tid] = sS[tid];
  if (w < D / 32) {
#pragma unroll
    for (int bi = 0; bi < D / 32; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        out[D + (size_t)(32 * bi + 8 * (i >> 2) + 4 * h + (i & 3)) * D + 32 * w + ln] = cacc[bi][i];
  }
}

// Ordered sum of a node's partials (same order on every run).
template <int D>
__global__ __launch_bounds__(256) void pddp_reduce_kernel(PddpParams p) {
  constexpr int E = D + D * D;
  constexpr int RB = (E + 255) / 256;
  const int bh = blockIdx.y, slot = blockIdx.x / RB;
  const int e = (blockIdx.x % RB) * 256 + threadIdx.x;
  const Node nd = pddp_node(slot, p.level, p.Nq, p.G);
  if (nd.c <= 1 || e >= E) return;
  const int parts = (nd.n + p.cr - 1) / p.cr;
  const size_t node = (size_t)bh * (1 << p.level) + slot;
  const double* src = p.part + node * p.pmax * E + e;
  // four partials loaded before they are added (four loads in flight), added in chunk order
  double s = 0.0;
  int q = 0;
  for (; q + 4 <= parts; q += 4) {
    double v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = src[(size_t)(q + i) * E];
#pragma unroll
    for (int i = 0; i < 4; ++i) s += v[i];
  }
  for (; q < parts; ++q) s += src[(size_t)q * E];
  p.red[node * E + e] = s;
}

template <int D>
__global__ __launch_bounds__(kNodeThreads) void pddp_power_kernel(PddpParams p) {
  constexpr int E = D + D * D;
  __shared__ double sS[D], sV[D], sY[2][D], sRed[2][4];
  const int bh = blockIdx.y, slot = blockIdx.x;
  const Node nd = pddp_node(slot, p.level, p.Nq, p.G);
  if (nd.c <= 1) return;
  const size_t node = (size_t)bh * (1 << p.level) + slot;
  const double* red = p.red + node * E;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
  double cacc[D / 32][16];
  if (tid < D) sS[tid] = red[tid];
  if (w < D / 32) {
#pragma unroll
    for (int bi = 0; bi < D / 32; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        cacc[bi][i] = red[D + (size_t)(32 * bi + 8 * (i >> 2) + 4 * h + (i & 3)) * D + 32 * w + ln];
  }
  __syncthreads();
  const double muv = centre_and_iterate<D>(cacc, sS, sV, sY, sRed, nd.n, p.iters);
  double* out = p.vec + node * (D + 1);
  if (tid < D) out[tid] = sV[tid];
  if (tid == 0) out[D] = muv;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void pddp_project_kernel(PddpParams p) {
  __shared__ double sV[D];
  __shared__ double s_muv;
  const int bh = blockIdx.y, slot = blockIdx.x / p.pj_pmax, chunk = blockIdx.x % p.pj_pmax;
  const Node nd = pddp_node(slot, p.level, p.Nq, p.G);
  if (nd.c <= 1) return;
  const int r0 = chunk * kProjRows;
  if (r0 >= nd.n) return;
  const int r1 = min(nd.n, r0 + kProjRows);
  const size_t node = (size_t)bh * (1 << p.level) + slot;
  const double* vec = p.vec + node * (D + 1);
  if ((int)threadIdx.x < D) sV[threadIdx.x] = vec[threadIdx.x];
  if (threadIdx.x == 0) s_muv = vec[D];
  __syncthreads();
  const double muv = s_muv;
  const size_t hbase = (size_t)bh * p.Nq;
  uint32_t* nkeys = p.keys + hbase + nd.start;
  project_rows<D, BF16, 256>(p.Q, hbase, p.perm + hbase + nd.start, r0, r1, sV, muv,
                             [&](int i, uint32_t k) { nkeys[i] = k; });
}

template <int NT, int VPT>
__global__ __launch_bounds__(NT) void pddp_split_kernel(PddpParams p) {
  using Sel = BlockSelect<NT, VPT>;
  __shared__ typename Sel::Shared sh;
  const int bh = blockIdx.y;
  const Node nd = pddp_node(blockIdx.x, p.level, p.Nq, p.G);
  if (nd.c <= 1) return;
  const size_t off = (size_t)bh * p.Nq + nd.start;
  int32_t* nperm = p.perm + off;
  int32_t* ntmp = p.tmp + off;
  const GlobalKeys keys{p.keys + off};
  const int nL = (nd.c >> 1) * p.G;
  Sel sel;
  sel.n = nd.n;
  sel.load(keys);
  uint32_t T;
  int tie_need;
  sel.threshold(keys, nL, sh, T, tie_need);
  // new position -> old position, then a batched gather through the key
  // array (no longer needed) and a copy back
  sel.split(keys, T, tie_need, sh, [&](int, int j, bool s, int pos) {
    const int dst = s ? pos : nL + pos;
    if (dst < nd.n) ntmp[dst] = j;
  });
  __syncthreads();
  int32_t* staged = (int32_t*)(p.keys + off);
  constexpr int U = 8;
  for (int i0 = 0; i0 < nd.n; i0 += U * NT) {
    int src[U], val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) src[u] = ntmp[min(i0 + u * NT + (int)threadIdx.x, nd.n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) val[u] = nperm[min(max(src[u], 0), nd.n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT + (int)threadIdx.x;
      if (i < nd.n) staged[i] = val[u];
    }
  }
  __syncthreads();
  for (int i0 = 0; i0 < nd.n; i0 += U * NT) {
    int val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) val[u] = staged[min(i0 + u * NT + (int)threadIdx.x, nd.n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT + (int)threadIdx.x;
      if (i < nd.n) nperm[i] = val[u];
    }
  }
}

__global__ void pddp_init_kernel(int32_t* perm, int Nq, size_t total) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < total) perm[i] = (int32_t)(i % (size_t)Nq);
}

// Host-side plan: the tree's shape depends only on Nq and G.
struct Plan {
  int levels, cr;
  size_t part, red, vec;  // doubles
};

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

long long level_max_rows(const Shape& s, int level) {
  const long long cmax = ((long long)s.c + (1LL << level) - 1) >> level;
  const long long n = cmax * s.G;
  return n < s.Nq ? n : s.Nq;
}

Plan make_plan(const Shape& s) {
  Plan pl{0, 0, 0, 0, 0};
  while ((1 << pl.levels) < s.c) ++pl.levels;
  long long cr = ((long long)s.BH * s.Nq + 511) / 512;
  cr = (cr + 63) / 64 * 64;
  pl.cr = (int)(cr < 2048 ? 2048 : (cr > kMaxChunkRows ? kMaxChunkRows : cr));
  const size_t E = (size_t)s.d + (size_t)s.d * s.d;
  for (int lv = 0; lv < pl.levels; ++lv) {
    const long long maxn = level_max_rows(s, lv);
    if (maxn <= pl.cr) break;
    const size_t nodes = (size_t)s.BH << lv;
    const size_t pmax = (size_t)((maxn + pl.cr - 1) / pl.cr);
    pl.part = std::max(pl.part, nodes * pmax * E);
    pl.red = std::max(pl.red, nodes * E);
    pl.vec = std::max(pl.vec, nodes * ((size_t)s.d + 1));
  }
  return pl;
}

template <int D, bool BF16>
void launch_levels(const Shape& s, const Plan& pl, PddpParams p, hipStream_t st) {
  constexpr int RB = (D + D * D + 255) / 256;
  for (int lv = 0; lv < pl.levels; ++lv) {
    p.level = lv;
    const int nslots = 1 << lv;
    const long long maxn = level_max_rows(s, lv);
    if (maxn > pl.cr) {
      p.pmax = (int)((maxn + pl.cr - 1) / pl.cr);
      const dim3 chunks(nslots * p.pmax, s.BH);
      hipLaunchKernelGGL((pddp_gram_kernel<D, BF16>), chunks, dim3(kNodeThreads), 0, st, p);
      hipLaunchKernelGGL((pddp_reduce_kernel<D>), dim3(nslots * RB, s.BH), dim3(256), 0, st, p);
      hipLaunchKernelGGL((pddp_power_kernel<D>), dim3(nslots, s.BH), dim3(kNodeThreads), 0, st, p);
      p.pj_pmax = (int)((maxn + kProjRows - 1) / kProjRows);
      hipLaunchKernelGGL((pddp_project_kernel<D, BF16>), dim3(nslots * p.pj_pmax, s.BH), dim3(256), 0, st, p);
      if (maxn <= 64LL * kSplitThreads)
        hipLaunchKernelGGL((pddp_split_kernel<kSplitThreads, 64>), dim3(nslots, s.BH), dim3(kSplitThreads), 0, st, p);
      else if (maxn <= 80LL * kSplitWideThreads)
        hipLaunchKernelGGL((pddp_split_kernel<kSplitWideThreads, 80>), dim3(nslots, s.BH), dim3(kSplitWideThreads), 0,
                           st, p);
      else
        hipLaunchKernelGGL((pddp_split_kernel<kSplitThreads, 0>), dim3(nslots, s.BH), dim3(kSplitThreads), 0, st, p);
    } else {
      const dim3 grid(nslots, s.BH);
      static_assert(kMaxChunkRows <= 16 * kNodeThreads, "node kernel register cache");
      if (BF16 && maxn <= kSmallRows)
        hipLaunchKernelGGL((pddp_small_kernel<D>), grid, dim3(kNodeThreads), 0, st, p);
      else if (maxn <= 2 * kNodeThreads)
        hipLaunchKernelGGL((pddp_node_kernel<D, BF16, 2>), grid, dim3(kNodeThreads), 0, st, p);
      else if (maxn <= 8 * kNodeThreads)
        hipLaunchKernelGGL((pddp_node_kernel<D, BF16, 8>), grid, dim3(kNodeThreads), 0, st, p);
      else
        hipLaunchKernelGGL((pddp_node_kernel<D, BF16, 16>), grid, dim3(kNodeThreads), 0, st, p);
    }
  }
}

}  // namespace

size_t pddp_workspace_bytes(const Shape& s) {
  const Plan pl = make_plan(s);
  const size_t n = (size_t)s.BH * s.Nq;
  return 2 * round256(n * 4) + round256(pl.part * 8) + round256(pl.red * 8) + round256(pl.vec * 8);
}

hipError_t launch_pddp(const Shape& s, bool bf16, const void* Q, int32_t* perm, void* ws, hipStream_t st) {
  const Plan pl = make_plan(s);
  const size_t n = (size_t)s.BH * s.Nq;
  char* w = (char*)ws;
  PddpParams p{};
  p.Q = Q;
  p.perm = perm;
  p.tmp = (int32_t*)w;
  w += round256(n * 4);
  p.keys = (uint32_t*)w;
  w += round256(n * 4);
  p.part = (double*)w;
  w += round256(pl.part * 8);
  p.red = (double*)w;
  w += round256(pl.red * 8);
  p.vec = (double*)w;
  p.Nq = s.Nq;
  p.G = s.G;
  p.iters = s.iters;
  p.cr = pl.cr;
  p.pmax = 1;
  hipLaunchKernelGGL(pddp_init_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, perm, s.Nq, n);
  if (bf16) {
    if (s.d == 128) launch_levels<128, true>(s, pl, p, st);
    else launch_levels<64, true>(s, pl, p, st);
  } else {
    if (s.d == 128) launch_levels<128, false>(s, pl, p, st);
    else launch_levels<64, false>(s, pl, p, st);
  }
  return hipGetLastError();
}

}  // namespace mcs
