// Fast-PDDP query grouping (MC-Sparse review, blog.secrett2633.cloud,
// section 3: similar queries are packed into equal-size, tile-aligned groups
// by Principal Direction Divisive Partitioning).
//
// The tree is processed level by level.  Groups are numbered depth-first, so
// every node is one contiguous range perm[start, start+n) of its head, and
// the node's shape (start, n, c groups) follows from its slot number alone.
// For a node with c >= 2 groups:
//   1. S = sum y and the scatter sum y y^T over the node's rows, where
//      y = x - r is the row shifted by a bf16 row r (bf16 inputs; fp32 inputs
//      use r = 0): the head's row 0 at the many-workgroup levels, the node's
//      first member row in pddp_node_kernel, the parent's mean row rounded
//      to bf16 in pddp_small_kernel; bf16 rows go through
//      v_mfma_f32_32x32x16_bf16 as y = hi + lo, two bf16 parts (exact
//      products, fp32 sums over 64-row tiles, fp64 across tiles), fp32 rows
//      with fp64 FMAs.  Without the shift, queries sharing a large mean would
//      make sum x x^T and S S^T / n nearly equal, and their fp32 sums would
//      lose the spread around the mean that the direction is taken from;
//   2. C = sum y y^T - S S^T / n (fp64, the same matrix as for x since
//      centring removes any shift; below the root the many-workgroup levels
//      form the sums of left children only and take a right child's as its
//      parent's minus its sibling's) and the fixed-step power iteration
//      v <- C v / ||C v|| from v0 = 1/sqrt(d) (a zero product keeps v): in
//      fp64 in pddp_node_kernel, in fp32 on C rounded to fp32 in
//      pddp_power_kernel and pddp_small_kernel, v normalised in fp64;
//   3. projections p_i = x_i . v - (r + S/n) . v in fp64, keyed by float(p_i);
//   4. the floor(c/2)*G members of smallest key, equal keys lowest position
//      first, go left, the rest right, both in their previous order (members
//      stay in ascending token order, so position order is index order).
//
// Two schedules.  Levels whose nodes are larger than `cr` rows (the top of
// the tree, few nodes) are spread over many workgroups: row chunks produce
// partial sums (step 1), an ordered reduction adds them, one workgroup per
// node iterates (step 2), row chunks project (step 3) and one workgroup per
// node splits (step 4, select.hpp).  Smaller nodes are done by one workgroup
// each from start to end, with the projection keys and member ids kept on
// chip (pddp_node_kernel, and pddp_small_kernel for nodes of at most 1024
// bf16 rows).
//
// In step 1 the gathered rows of a tile (64 rows; 32 in the small-node
// kernel) are copied straight into LDS (global_load_lds, 16 bytes per lane)
// in a ring of two slots (pddp_node_kernel) or three, row-major with the
// 16-byte chunks XOR-swizzled per row; both MFMA operands (x^T blocks) are
// read with ds_read_b64_tr_b16.  The scatter matrix is symmetric, so only
// the blocks of one triangle are formed (ten of sixteen 32x32 blocks at
// d = 128, three of four at d = 64), spread over the waves; the chunks of
// the many-workgroup levels are sized per level (gram_chunk_rows).  For the
// power iteration wave w holds column block w of C in the MFMA output layout
// (lane: one column, 16 rows per 32-row block), so C v needs only an in-lane
// sum and one half-wave exchange.
#include <algorithm>
#include <type_traits>

#include "mcs_kernels.hpp"
#include "ring.hpp"
#include "select.hpp"

namespace mcs {
namespace {

constexpr int kNodeThreads = 256;
constexpr int kSplitThreads = 512;
constexpr int kSplitWideThreads = 1024;  // nodes of more than 8192 rows
constexpr int kProjRows = 512;      // rows per workgroup of the projection kernel
constexpr int kMaxChunkRows = 4096;  // row chunk of the many-workgroup levels; larger nodes split there

struct PddpParams {
  const void* Q;
  int32_t* perm;
  int32_t* tmp;
  uint32_t* keys;
  double* part;  // [BH][nslots][pmax][D + D*D] partial (S, sum x x^T) per row chunk
  double* red;       // [BH][nslots][D + D*D] their sums at this level
  double* red_prev;  // the same at the level above (many-workgroup levels below the root)
  __bf16* mean_cur;          // [BH][nslots][D] each node's mean row rounded to bf16 (bf16 inputs)
  const __bf16* mean_prev;   // the same at the level above: the small-node kernel's shift
  double* vec;   // [BH][nslots][D + 1] direction v and (S/n) . v
  int Nq, G, iters, level, cr, pmax;
  int cg;       // rows per partial scatter sum (a chunk of a node) at the many-workgroup levels
  int pj_pmax;  // projection chunks (of kProjRows rows) per node at this level
};

struct Node {
  int start, n, c;
};

// y = x - r as two bf16 parts, hi = bf16(y) and lo = bf16(y - hi).  x and r
// are bf16 values, so y and y - hi are exact in fp32 and hi + lo equals y
// whenever y has at most 16 significant bits (otherwise it is within 2^-17
// of y); products of the parts are exact in the fp32 MFMA accumulators.
__device__ __forceinline__ void split_shifted(bf16x8 x, float r, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float y = (float)x[j] - r;
    const __bf16 h = (__bf16)y;
    hi[j] = h;
    lo[j] = (__bf16)(y - (float)h);
  }
}

// The rows of an LDS tile (ring.hpp layout: row-major, 16-byte chunks
// XOR-swizzled per row) shifted by r and split in place: each chunk x of 8
// channels becomes hi = bf16(x - r), and the chunk at the same offset of `lo`
// becomes bf16(x - r - hi) (split_shifted).  Each element is split once, by
// one thread; the MFMA operands are then read from both tiles as they are.
template <int D, int ROWS, int NT>
__device__ __forceinline__ void split_tile(unsigned char* slot, unsigned char* lo, const float* sRf) {
  constexpr int CH = D / 8;
  static_assert((ROWS * CH) % NT == 0, "chunks per thread");
#pragma unroll 1
  for (int k = 0; k < ROWS * CH / NT; ++k) {
    const int ci = k * NT + (int)threadIdx.x;
    const int row = ci / CH, pos = ci % CH;
    const int ch = 8 * (pos ^ swz<D>(row));  // first channel of the chunk
    bf16x8* px = (bf16x8*)(slot + row * (2 * D) + 16 * pos);
    const bf16x8 x = *px;
    const f32x4 ra = *(const f32x4*)(sRf + ch), rb = *(const f32x4*)(sRf + ch + 4);
    bf16x8 h, l;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float y = (float)x[j] - (j < 4 ? ra[j] : rb[j - 4]);
      const __bf16 hj = (__bf16)y;
      h[j] = hj;
      l[j] = (__bf16)(y - (float)hj);
    }
    *px = h;
    *(bf16x8*)(lo + row * (2 * D) + 16 * pos) = l;
  }
}

// Row `tid` < D of a node's mean, r + S/n (S: the sums of the rows shifted
// by r), rounded to bf16: the children's shift in the small-node kernel.
template <int D>
__device__ __forceinline__ void store_mean(const PddpParams& p, int bh, int slot, const double* sR, const double* sS,
                                           int n) {
  const int tid = threadIdx.x;
  if (tid < D)
    p.mean_cur[(((size_t)bh << p.level) + slot) * D + tid] = (__bf16)(sR[tid] + sS[tid] / (double)n);
}

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
  static constexpr int SLOT2 = BF16 ? GramCfg<D>::TILE_BYTES : 16;
  static constexpr int SLOTLO = BF16 ? GramCfg<D>::TILE_BYTES : 16;  // low parts of the split tile
};

// Step 1 over member rows [r0, r1) of a node (nperm: the node's members).
// cacc (waves w < NB): sum y y^T, element (bi, i) = row 32*bi + 8*(i/4) +
// 4*h + i%4, column 32*w + lane%32.  sS[0..D): sum y.  For bf16 rows
// y = x - Q[shift] (a row of the head: the node's first member row in the
// node kernel, the head's row 0 at the many-workgroup levels), for fp32 rows
// y = x.  Ends with a barrier.
// Partial sums of the many-workgroup levels: S (D doubles), then the
// scatter matrix.  bf16 rows at d = 128 form only the ten blocks of one
// triangle (gram_rows), stored as ten 32x32 blocks in the MFMA output layout
// (element i of lane l at i*64 + l): block m = W is (W, W), m = 4 + W is
// (W+1 mod 4, W), m = 8 + W is (W+2, W) for W < 2 (rows, columns).  Other
// inputs store the full matrix, row-major.
template <int D, bool BF16>
constexpr bool kSymPart = BF16 && D == 128;
template <int D, bool BF16>
constexpr int kPartE = kSymPart<D, BF16> ? D + 10 * 1024 : D + D * D;

template <int D, bool BF16, int NS, bool XCH = true>
__device__ void gram_rows(const void* Qv, size_t hbase, const int32_t* nperm, int r0, int r1, int shift,
                          unsigned char* slot0, unsigned char* slot1, unsigned char* slot2, unsigned char* slotlo,
                          float* sRf, double (&cacc)[D / 32][16], double* sS) {
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
    // the shift r: row `shift` of the head, in LDS as float32 (published by
    // the first barrier of the tile loop)
    if (tid < D) sRf[tid] = (float)Qh[(size_t)shift * D + tid];
    // column sums: lane (n, h) of wave w keeps element n%16 of the ones-product,
    // i.e. S[32w + 8((n%16)/4) + 4h + n%4]
    double sacc = 0.0;
    const int si = ln & 15;
    // member ids of the tile to be copied next (loaded a tile before its copy is issued)
    int ids[C::LPW];
    auto load_ids = [&](int t) {
#pragma unroll
      for (int j = 0; j < C::LPW; ++j) {
        const int r = C::RPL * (w + 4 * j) + lrow0;
        const int i = r0 + t * 64 + r;
        ids[j] = i < r1 ? nperm[i] : shift;  // tail rows: the shift row, which shifts to exactly 0
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
    // y^T operand of channel block b for 16-row step ks2 from a split tile (hi or lo part)
    auto operand = [&](const unsigned char* t, int b, int ks2) {
      const unsigned char* base = t + 16 * (2 * D) * ks2;
      return cat(lds_read_tr(base + (ob0 ^ (64 * b))), lds_read_tr(base + (ob1 ^ (64 * b))));
    };
    // one fp32 accumulator live at a time (row blocks outer), which keeps the
    // kernel within 256 registers per lane (a chain of dependent MFMAs issues
    // as fast as independent ones); y y^T = (hi + lo)(hi + lo)^T as four exact
    // products.  Block (a, c): rows of channel block a, columns of block c.
    auto block = [&](const unsigned char* slot, int a, int c, bool sums, f32x16& accS) {
      f32x16 acc = {};
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2) {
        const bf16x8 wh = operand(slot, c, ks2), wl = operand(slotlo, c, ks2);
        const bf16x8 hb = operand(slot, a, ks2), lb = operand(slotlo, a, ks2);
        acc = mfma_32x32x16(hb, wh, acc);
        acc = mfma_32x32x16(hb, wl, acc);
        acc = mfma_32x32x16(lb, wh, acc);
        acc = mfma_32x32x16(lb, wl, acc);
        if (sums) {
          accS = mfma_32x32x16(wh, ones, accS);
          accS = mfma_32x32x16(wl, ones, accS);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) cacc[a][i] += (double)acc[i];
    };
    auto add_sums = [&](const f32x16& accS) {
      float sv = accS[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) sv = (si == i) ? accS[i] : sv;
      sacc += (double)sv;
    };
    // d = 128: the matrix is symmetric, so only ten of its sixteen blocks are
    // formed: wave W the blocks (W, W), (W+1, W) and, for W < 2, (W+2, W)
    // (indices mod 4), all in its own column; the blocks of its column formed
    // by other waves arrive transposed through LDS after the last tile
    auto compute_sym = [&](const unsigned char* slot, auto wc) {
      constexpr int W = decltype(wc)::value;
      f32x16 accS = {};
      block(slot, W, W, true, accS);
      block(slot, (W + 1) & 3, W, false, accS);
      if constexpr (W < 2) block(slot, W + 2, W, false, accS);
      add_sums(accS);
    };
    static_assert(NS == 2 || NS == 3, "ring depth");
    unsigned char* const ring[3] = {slot0, slot1, slot2};
    // Tile t lands in ring slot t % NS by direct-to-LDS copies issued NS-1
    // tiles ahead; after a barrier it is split in place (the low parts in
    // slotlo, single-buffered: every wave has finished the previous tile at
    // that barrier), then, after another, used.  Per tile a wave issues LPW
    // copies and then LPW id loads, so when tile t is waited for, the loads
    // issued after its copies are ids(t+1) and, per later tile in flight, its
    // copies and the next ids: (2 NS - 3) LPW in all.
    for (int k = 0; k < NS - 1 && k < ntiles; ++k) {
      load_ids(k);
      issue(ring[k]);
    }
    if (NS - 1 < ntiles) load_ids(NS - 1);
    // unrolled by NS so that every slot address is a constant of its copy
    auto tiles = [&](auto cf) {
      for (int t0 = 0; t0 < ntiles; t0 += NS) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          const int t = t0 + k;
          if (t >= ntiles) break;
          if (t + NS - 1 < ntiles) wait_vmcnt<(2 * NS - 3) * C::LPW>();
          else wait_vmcnt<0>();
          __syncthreads();
          if (t + NS - 1 < ntiles) {
            issue(ring[(k + NS - 1) % NS]);  // the slot of tile t-1, whose last reads ended before the barrier
            if (t + NS < ntiles) load_ids(t + NS);
          }
          split_tile<D, 64, 256>(ring[k], slotlo, sRf);
          __syncthreads();
          cf(ring[k]);
        }
      }
    };
    if constexpr (NB == 4) {
      // 32x32 fp64 blocks exchanged through the tile slots (free after the
      // last tile): block m holds wave m's (m+1, m) block for m < 4 and wave
      // m-4's (m-2, m-4) block for m = 4, 5; element (r, c) at r*32 + (c ^ r)
      // (conflict-free both for the row-wise stores and the column-wise reads)
      auto xblk = [&](int m) {
        return (double*)(m < 2 ? slot0 + m * 8192 : (m < 4 ? slot1 + (m - 2) * 8192 : slotlo + (m - 4) * 8192));
      };
      auto run = [&](auto wc) {
        constexpr int W = decltype(wc)::value;
        tiles([&](const unsigned char* slot) { compute_sym(slot, wc); });
        if constexpr (!XCH) return;  // the caller stores the formed blocks as they are
        __syncthreads();  // every operand read of the last tile is done
        auto put = [&](int m, int a) {
          double* X = xblk(m);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 8 * (i >> 2) + 4 * h + (i & 3);
            X[r * 32 + (ln ^ r)] = cacc[a][i];
          }
        };
        put(W, (W + 1) & 3);
        if constexpr (W < 2) put(4 + W, W + 2);
        __syncthreads();
        // block (bi, W) of this column is the transpose of block (W, bi),
        // formed by wave bi
        auto get = [&](int m, int bi) {
          const double* X = xblk(m);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 8 * (i >> 2) + 4 * h + (i & 3);
            cacc[bi][i] = X[ln * 32 + (r ^ ln)];
          }
        };
        if constexpr (W == 0) get(3, 3);
        if constexpr (W == 1) get(0, 0);
        if constexpr (W == 2) {
          get(4, 0);
          get(1, 1);
        }
        if constexpr (W == 3) {
          get(5, 1);
          get(2, 2);
        }
      };
      switch (__builtin_amdgcn_readfirstlane(w)) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        default: run(std::integral_constant<int, 3>{}); break;
      }
    } else {
      // d = 64: three of the four blocks, one per wave: (0, 0) by wave 0,
      // (1, 1) by wave 1, (1, 0) by wave 2, which passes it through the first
      // tile slot (layout as above) to wave 0 as it is and to wave 1
      // transposed; wave 3 only copies and splits tiles
      auto run = [&](auto wc) {
        constexpr int W = decltype(wc)::value;
        tiles([&](const unsigned char* slot) {
          f32x16 accS = {};
          if constexpr (W < 2) {
            block(slot, W, W, true, accS);
            add_sums(accS);
          } else if constexpr (W == 2) {
            block(slot, 1, 0, false, accS);
          }
        });
        double* X = (double*)slot0;
        __syncthreads();  // every operand read of the last tile is done
        if constexpr (W == 2) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 8 * (i >> 2) + 4 * h + (i & 3);
            X[r * 32 + (ln ^ r)] = cacc[1][i];
          }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * h + (i & 3);
          if constexpr (W == 0) cacc[1][i] = X[r * 32 + (ln ^ r)];
          if constexpr (W == 1) cacc[0][i] = X[ln * 32 + (r ^ ln)];
        }
      };
      switch (__builtin_amdgcn_readfirstlane(w)) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        default: run(std::integral_constant<int, 3>{}); break;
      }
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

// Step 2.  cacc holds sum y y^T (layout of gram_rows), sS the column sums
// of y = x - r and sR the shift r (NULL: r = 0), both visible to all
// threads.  Leaves v in sV and returns the node mean's projection
// (r + S/n) . v.
// With v_k = y_k / ||y_k||, the iteration runs as y_{k+1} = C y_k / ||y_k||:
// the norm of y_k is reduced while y_{k+1} is formed, so one barrier per step
// suffices (y double-buffered in sY).  If C v_k = 0 the direction stays v_k.
// Sum over the 64 lanes, in every lane: DPP within rows of 16, then the
// 16-lane and 32-lane half swaps (no LDS permutes).
__device__ __forceinline__ double wave_sum16_f64(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const auto lo = __builtin_amdgcn_permlane16_swap((unsigned)u, (unsigned)u, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
  // r[0] + r[1]: the even row's value plus the odd row's, in both rows
  v = __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0])) +
      __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
  return v + partner32_f64(v);
}

template <int D, int YB>
__device__ double centre_and_iterate(double (&cacc)[D / 32][16], const double* sS, const double* sR, double* sV,
                                     double (*sY)[D], double (*sRed)[4], int n, int iters) {
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
    // this lane's rows of y_k, read YB row blocks at a time before they are
    // used (the reads' latencies overlap; YB < NB bounds the registers)
    static_assert(NB % YB == 0, "row blocks per read batch");
    double2 yv[YB][8];
    auto read_y = [&](int b0) {
#pragma unroll
      for (int j = 0; j < YB; ++j)
#pragma unroll
        for (int g = 0; g < 8; ++g) yv[j][g] = *(const double2*)&sY[cur][(b0 + j) * 32 + 8 * (g >> 1) + 4 * h + 2 * (g & 1)];
    };
    if (gw) read_y(0);
    const double nrm2 = (sRed[cur][0] + sRed[cur][1]) + (sRed[cur][2] + sRed[cur][3]);
    if (nrm2 == 0.0) break;  // C v = 0: keep the previous direction
    last = cur;
    const double inv = __builtin_amdgcn_rsq(nrm2);  // any scale serves: the direction is scale-free
    double wv = 0.0;
    if (gw) {
      double part[NB];  // independent FMA chains, one per row block
#pragma unroll
      for (int b0 = 0; b0 < NB; b0 += YB) {
        if (b0) read_y(b0);
#pragma unroll
        for (int j = 0; j < YB; ++j) {
          part[b0 + j] = 0.0;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const double2 y2 = yv[j][i >> 1];
            part[b0 + j] = fma(cacc[b0 + j][i], (i & 1) ? y2.y : y2.x, part[b0 + j]);
          }
        }
      }
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) wv += part[bi];
      wv += partner32_f64(wv);
      wv *= inv;
    }
    const double sq = wave_sum16_f64((gw && h == 0) ? wv * wv : 0.0);
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
  const double mv = wave_sum_f64(tid < D ? ((sR ? sR[tid] : 0.0) + sS[tid] * inv_n) * sV[tid] : 0.0);
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
    // sum over the row's LPR lanes (8 or 16, aligned) by DPP moves: quad
    // swaps, then the half-row and row mirrors (every lane of a quad holds the
    // same quad sum, so a mirror adds the same value an xor 4 / xor 8
    // exchange would: the keys equal those of a shuffle reduction bit for bit)
    static_assert(LPR == 8 || LPR == 16, "lanes per row");
    d += dpp_f64<0xB1>(d);  // quad_perm [1,0,3,2]
    d += dpp_f64<0x4E>(d);  // quad_perm [2,3,0,1]
    d += dpp_f64<0x141>(d);  // row_half_mirror
    if constexpr (LPR == 16) d += dpp_f64<0x140>(d);  // row_mirror
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
  constexpr int U = 8;  // rows per lane group in flight
  const int w = wave_id(), sub = lane_id() / P::LPR;
  const int step = NT / 64 * P::RPW;
  // the member ids of the next batch are loaded while this batch's rows are
  // in flight, so each batch waits for one memory latency, not two
  int id[U];
  const int b0 = r0 + w * P::RPW;
#pragma unroll
  for (int u = 0; u < U; ++u) id[u] = nperm[min(b0 + u * step + sub, r1 - 1)];
  for (int b = b0; b < r1; b += U * step) {
    typename P::Row x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = pr.load(Qv, hbase + id[u]);
    const int bn = b + U * step;
    if (bn < r1) {
#pragma unroll
      for (int u = 0; u < U; ++u) id[u] = nperm[min(bn + u * step + sub, r1 - 1)];
    }
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
  __shared__ __attribute__((aligned(1024))) unsigned char slotlo[L::SLOTLO];
  __shared__ __attribute__((aligned(16))) float sRf[D];
  __shared__ double sS[D], sR[D], sV[D], sRed[2][4];
  __shared__ __attribute__((aligned(16))) double sY[2][D];
  __shared__ typename Sel::Shared sh;
  // the projection keys reuse the first tile slot once the scatter sums are
  // done (when they fit: d = 128)
  constexpr bool kKeysInSlot = VPT * kNodeThreads * 4 <= L::SLOT0;
  __shared__ uint32_t s_keys_own[kKeysInSlot ? 1 : VPT * kNodeThreads];
  uint32_t* const s_keys = kKeysInSlot ? (uint32_t*)slot0 : s_keys_own;
  const int bh = blockIdx.y;
  const Node nd = pddp_node(blockIdx.x, p.level, p.Nq, p.G);
  if (nd.c <= 1) return;
  const size_t hbase = (size_t)bh * p.Nq;
  int32_t* nperm = p.perm + hbase + nd.start;
  if (BF16 && (int)threadIdx.x < D) sR[threadIdx.x] = (double)(float)((const __bf16*)p.Q)[(hbase + nperm[0]) * D + threadIdx.x];
  double cacc[D / 32][16];
  gram_rows<D, BF16, 2>(p.Q, hbase, nperm, 0, nd.n, nperm[0], slot0, slot1, slot1, slotlo, sRf, cacc,
                        sS);  // its final barrier publishes sR
  if constexpr (BF16) store_mean<D>(p, bh, blockIdx.x, sR, sS, nd.n);
  const double muv = centre_and_iterate<D, D / 64>(cacc, sS, BF16 ? sR : nullptr, sV, sY, sRed, nd.n, p.iters);
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

// The fixed-step power iteration in fp32 on C held in the MFMA output layout
// (cf, waves w < D/32: column block w), from v0 = 1/sqrt(d); the direction,
// normalised in fp64, goes to sV.  Ends with a barrier.
template <int D>
__device__ __forceinline__ void power_f32(const float (&cf)[D / 32][16], float (*sY)[D], double* sV, int iters) {
  constexpr int NB = D / 32;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
  const bool gw = w < NB;
  if (tid < D) sY[0][tid] = 1.0f / sqrtf((float)D);
  __syncthreads();
  // Every lane reads the rows 8g + 4h + 0..3 of each 32-row block of y for
  // C y.  ||y||^2 is formed by every wave alike, so no reduction across waves
  // is needed: each lane squares entries l and l + 64, then a sum over the
  // wave by DPP moves and two lane-half swaps (every lane ends with the same
  // bits).  The step's scale 1/||y_k|| uses the hardware reciprocal square
  // root (the direction does not depend on the scale; v is normalised in fp64
  // below).
  auto norm2 = [&](int buf) {
    const float y0 = sY[buf][l];
    float q = y0 * y0;
    if constexpr (D > 64) {
      const float y1 = sY[buf][l + 64];
      q = fmaf(y1, y1, q);
    }
    q += dpp_f32<0xB1>(q);   // quad_perm [1,0,3,2]
    q += dpp_f32<0x4E>(q);   // quad_perm [2,3,0,1]
    q += dpp_f32<0x141>(q);  // row_half_mirror
    q += dpp_f32<0x140>(q);  // row_mirror
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(q), __float_as_uint(q), false, false);
    q = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);  // rows 0+1, 2+3 of 16 lanes
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(q), __float_as_uint(q), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
  };
  int cur = 0, last = 0;
  float nl = 1.0f;  // ||y_last||^2
  for (int it = 0; it < iters; ++it) {
    const float nrm2 = norm2(cur);
    if (nrm2 == 0.0f) break;  // C v = 0: keep the previous direction
    last = cur;
    nl = nrm2;
    const float inv = __builtin_amdgcn_rsqf(nrm2);
    float wv = 0.0f;
    if (gw) {
      // y read two row blocks at a time (fewer registers: four workgroups per CU)
      float part[NB];
#pragma unroll
      for (int b0 = 0; b0 < NB; b0 += 2) {
        f32x4 yv[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) yv[j][g] = *(const f32x4*)&sY[cur][(b0 + j) * 32 + 8 * g + 4 * h];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          part[b0 + j] = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) part[b0 + j] = fmaf(cf[b0 + j][i], yv[j][i >> 2][i & 3], part[b0 + j]);
        }
      }
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) wv += part[bi];
      wv = half_sum(wv) * inv;
    }
    const int nxt = cur ^ 1;
    if (gw && h == 0) sY[nxt][w * 32 + ln] = wv;
    __syncthreads();
    cur = nxt;
  }
  {
    const float nrm2 = norm2(cur);
    if (nrm2 != 0.0f) {
      last = cur;
      nl = nrm2;
    }
  }
  const double vinv = 1.0 / sqrt((double)nl);
  if (tid < D) sV[tid] = (double)sY[last][tid] * vinv;
  __syncthreads();
}

// ---- small nodes ------------------------------------------------------------
// Nodes of at most kSmallRows rows (the deep levels: thousands of nodes, each a
// chain of latencies) run with a lighter state so that four workgroups share
// a CU (at d = 128: 128 registers, with a few spills in the one-time
// centring, and 39 KB of LDS): the scatter sums of the shifted
// rows y = x - r (r: the parent's mean row rounded to bf16, the first member
// row at the root; y = hi + lo in two bf16 parts, see split_shifted) stay in
// the fp32 MFMA accumulators over all tiles
// (exact products, fp32 sums over at most kSmallRows rows), the centring is
// done in fp64 and the power iteration runs in fp32 (C rounded to fp32); the
// projections stay fp64.  Row tiles of 32 rows in a three-slot ring.
constexpr int kSmallRows = 1024;

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
  // at d = 128 the block select's tables share the ring slots, which are
  // free once the scatter sums are formed (39 KB of LDS: four workgroups per
  // CU instead of two)
  constexpr bool kShInSlots = sizeof(typename Sel::Shared) <= 3 * TILE;
  __shared__ __attribute__((aligned(1024))) unsigned char slots[3 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char slotlo[TILE];
  __shared__ typename Sel::Shared sh_own[1];  // d = 64 only (removed when unused)
  unsigned char* const slot0 = slots;
  unsigned char* const slot1 = slots + TILE;
  unsigned char* const slot2 = slots + 2 * TILE;
  typename Sel::Shared& sh = kShInSlots ? *reinterpret_cast<typename Sel::Shared*>(slots) : sh_own[0];
  __shared__ __attribute__((aligned(16))) float sRf[D];
  __shared__ double sS[D], sR[D], sV[D], sMu[4];
  __shared__ __attribute__((aligned(16))) float sY[2][D];
  // the projection keys in the low-part slot, free once the scatter is formed
  static_assert(kSmallRows * 4 <= TILE, "keys in the low-part slot");
  uint32_t* const s_keys = (uint32_t*)slotlo;
  const int bh = blockIdx.y;
  const Node nd = pddp_node(blockIdx.x, p.level, p.Nq, p.G);
  if (nd.c <= 1) return;
  const size_t hbase = (size_t)bh * p.Nq;
  int32_t* nperm = p.perm + hbase + nd.start;
  const int n = nd.n;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const bool gw = w < NB;

  // ---- 1. scatter sums of the shifted rows, fp32 over all tiles ---------------
  const __bf16* Qh = (const __bf16*)p.Q + hbase * D;
  // the shift r: the parent's mean row (bf16) below the root, else the first
  // member row; published by the tile loop's first barrier.  (With the first
  // member row the column-mean part of the sums dwarfs the scatter and the
  // fp32 sums over the tiles moved the projections by up to four times the
  // parity band on a few nodes in a hundred; shifted by the parent's mean
  // they stay within a fraction of it.)
  const __bf16* rrow =
      p.level > 0 ? p.mean_prev + (((size_t)bh << (p.level - 1)) + (blockIdx.x >> 1)) * D : Qh + (size_t)nperm[0] * D;
  if (tid < D) {
    sR[tid] = (double)(float)rrow[tid];
    sRf[tid] = (float)rrow[tid];
  }
  const int vr = 4 * h + ((l & 15) >> 2);
  const int c0 = 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
  const int ob0 = vr * (2 * D) + 8 * (l & 1) + 16 * (c0 ^ swz<D>(vr));
  const int ob1 = (8 + vr) * (2 * D) + 8 * (l & 1) + 16 * (c0 ^ swz<D>(8 + vr));
  const int lrow0 = l / CH, lchunk = l % CH;
  const int ntiles = (n + TR - 1) / TR;
  int ids[LPW];
  auto load_ids = [&](int t) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int i = t * TR + RPL * (wu + 4 * j) + lrow0;
      ids[j] = i < n ? nperm[i] : -1;  // tail rows: the shift itself, which shifts to exactly 0
    }
  };
  auto issue = [&](unsigned char* slot) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int r = RPL * (wu + 4 * j) + lrow0;
      dma16((ids[j] >= 0 ? Qh + (size_t)ids[j] * D : rrow) + ((lchunk ^ swz<D>(r)) * 8), slot + (wu + 4 * j) * 1024);
    }
  };
  bf16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (__bf16)1.0f;
  f32x16 acc[NB], accS = {};
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
  // y^T operands from the split tile (hi part in the slot, lo part in slotlo);
  // the blocks (a, c) with a in rows, c in columns, formed for every a in `as`
  auto compute_blocks = [&](const unsigned char* slot, int c, bool sums, auto... as) {
#pragma unroll
    for (int ks2 = 0; ks2 < TR / 16; ++ks2) {
      auto part = [&](const unsigned char* t, int b) {
        const unsigned char* base = t + 16 * (2 * D) * ks2;
        return cat(lds_read_tr(base + (ob0 ^ (64 * b))), lds_read_tr(base + (ob1 ^ (64 * b))));
      };
      const bf16x8 wh = part(slot, c), wl = part(slotlo, c);  // the column block
      auto one = [&](int bi) {
        const bf16x8 hb = part(slot, bi), lb = part(slotlo, bi);
        acc[bi] = mfma_32x32x16(hb, wh, acc[bi]);
        acc[bi] = mfma_32x32x16(hb, wl, acc[bi]);
        acc[bi] = mfma_32x32x16(lb, wh, acc[bi]);
        acc[bi] = mfma_32x32x16(lb, wl, acc[bi]);
      };
      (one(as), ...);
      if (sums) {
        accS = mfma_32x32x16(wh, ones, accS);
        accS = mfma_32x32x16(wl, ones, accS);
      }
    }
  };
  // Tile t lands in slot t % 3 by copies issued two tiles ahead (ids loaded a
  // tile before their copies); after a barrier it is split in place (low
  // parts in slotlo, single-buffered: every wave has finished the previous
  // tile at that barrier), then, after another, used.  When tile t is waited
  // for, the loads issued after its copies are ids(t+1), the copies of t+1
  // and ids(t+2).
  unsigned char* const ring[3] = {slot0, slot1, slot2};
  load_ids(0);
  issue(ring[0]);
  if (ntiles > 1) {
    load_ids(1);
    issue(ring[1]);
    if (ntiles > 2) load_ids(2);
  }
  auto tiles = [&](auto cf) {
    for (int t0 = 0; t0 < ntiles; t0 += 3) {
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int t = t0 + k;
        if (t >= ntiles) break;
        if (t + 2 < ntiles) wait_vmcnt<3 * LPW>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (t + 2 < ntiles) {
          issue(ring[(k + 2) % 3]);  // the slot of tile t-1, whose last reads ended before the barrier
          if (t + 3 < ntiles) load_ids(t + 3);
        }
        split_tile<D, TR, kNodeThreads>(ring[k], slotlo, sRf);
        __syncthreads();
        cf(ring[k]);
      }
    }
  };
  if constexpr (NB == 4) {
    // d = 128: the scatter matrix is symmetric, so wave W forms only the
    // blocks (W, W), (W+1, W) and, for W < 2, (W+2, W) (indices mod 4) of its
    // column; the other blocks of its column arrive transposed through the
    // tile slots after the last tile (fp32 32x32 blocks, element (r, c) at
    // r*32 + (c ^ r): block m holds wave m's (m+1, m) block for m < 4 and
    // wave m-4's (m-2, m-4) block for m = 4, 5)
    auto xblk = [&](int m) { return (float*)(m < 4 ? ring[m >> 1] + (m & 1) * 4096 : slotlo + (m - 4) * 4096); };
    auto run = [&](auto wc) {
      constexpr int W = decltype(wc)::value;
      if constexpr (W < 2) tiles([&](const unsigned char* slot) { compute_blocks(slot, W, true, W, (W + 1) & 3, W + 2); });
      else tiles([&](const unsigned char* slot) { compute_blocks(slot, W, true, W, (W + 1) & 3); });
      __syncthreads();  // every operand read of the last tile is done
      auto put = [&](int m, int a) {
        float* X = xblk(m);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * h + (i & 3);
          X[r * 32 + (ln ^ r)] = acc[a][i];
        }
      };
      put(W, (W + 1) & 3);
      if constexpr (W < 2) put(4 + W, W + 2);
      __syncthreads();
      auto get = [&](int m, int bi) {
        const float* X = xblk(m);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * h + (i & 3);
          acc[bi][i] = X[ln * 32 + (r ^ ln)];
        }
      };
      if constexpr (W == 0) get(3, 3);
      if constexpr (W == 1) get(0, 0);
      if constexpr (W == 2) {
        get(4, 0);
        get(1, 1);
      }
      if constexpr (W == 3) {
        get(5, 1);
        get(2, 2);
      }
    };
    switch (wu) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      default: run(std::integral_constant<int, 3>{}); break;
    }
  } else {
    // d = 64: (0, 0) by wave 0, (1, 1) by wave 1, (1, 0) by wave 2, passed
    // through the first slot to wave 0 as it is and to wave 1 transposed
    auto run = [&](auto wc) {
      constexpr int W = decltype(wc)::value;
      tiles([&](const unsigned char* slot) {
        if constexpr (W < 2) compute_blocks(slot, W, true, W);
        else if constexpr (W == 2) compute_blocks(slot, 0, false, 1);
      });
      float* X = (float*)slot0;
      __syncthreads();  // every operand read of the last tile is done
      if constexpr (W == 2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * h + (i & 3);
          X[r * 32 + (ln ^ r)] = acc[1][i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * h + (i & 3);
        if constexpr (W == 0) acc[1][i] = X[r * 32 + (ln ^ r)];
        if constexpr (W == 1) acc[0][i] = X[ln * 32 + (r ^ ln)];
      }
    };
    switch (wu) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      default: run(std::integral_constant<int, 3>{}); break;
    }
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
  store_mean<D>(p, bh, blockIdx.x, sR, sS, n);

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
  power_f32<D>(cf, sY, sV, p.iters);
  const double mv = wave_sum_f64(tid < D ? (sR[tid] + sS[tid] * inv_n) * sV[tid] : 0.0);
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
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[L::SLOT2];
  __shared__ __attribute__((aligned(1024))) unsigned char slotlo[L::SLOTLO];
  __shared__ __attribute__((aligned(16))) float sRf[D];
  __shared__ double sS[D];
  // below the root only left children (even slots) are summed: a right
  // child's sums are its parent's minus its sibling's (pddp_reduce_kernel);
  // every node of these levels is shifted by the head's row 0, so that the
  // sums of parent and children share the shift
  const int below = p.level > 0;
  const int bh = blockIdx.y, slot = (blockIdx.x / p.pmax) << below, chunk = blockIdx.x % p.pmax;
  const Node nd = pddp_node(slot, p.level, p.Nq, p.G);
  if (nd.c <= 1 - below) return;  // the root: split only if c > 1; a left child: needed whenever it exists
  const int r0 = chunk * p.cg;
  if (r0 >= nd.n) return;
  const int r1 = min(nd.n, r0 + p.cg);
  const size_t hbase = (size_t)bh * p.Nq;
  double cacc[D / 32][16];
  constexpr int E = kPartE<D, BF16>;
  gram_rows<D, BF16, 3, !kSymPart<D, BF16>>(p.Q, hbase, p.perm + hbase + nd.start, r0, r1, 0, slot0, slot1, slot2,
                                            slotlo, sRf, cacc, sS);
  const int nslots = 1 << p.level;
  double* out = p.part + (((size_t)bh * nslots + slot) * p.pmax + chunk) * E;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
  if (tid < D) out[tid] = sS[tid];
  if constexpr (kSymPart<D, BF16>) {
    // the blocks this wave formed (see kPartE)
    auto put = [&](int m, int a) {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[D + m * 1024 + i * 64 + l] = cacc[a][i];
    };
    switch (__builtin_amdgcn_readfirstlane(w)) {
      case 0: put(0, 0); put(4, 1); put(8, 2); break;
      case 1: put(1, 1); put(5, 2); put(9, 3); break;
      case 2: put(2, 2); put(6, 3); break;
      default: put(3, 3); put(7, 0); break;
    }
  } else if (w < D / 32) {
#pragma unroll
    for (int bi = 0; bi < D / 32; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        out[D + (size_t)(32 * bi + 8 * (i >> 2) + 4 * h + (i & 3)) * D + 32 * w + ln] = cacc[bi][i];
  }
}

// Ordered sum of a node's partials (same order on every run).  Below the
// root the workgroups of a left child also form its sibling's sums: its
// parent's sums minus the left child's (one fp64 rounding).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void pddp_reduce_kernel(PddpParams p) {
  constexpr int E = kPartE<D, BF16>;
  constexpr int RB = (E + 255) / 256;
  const int below = p.level > 0;
  const int bh = blockIdx.y, slot = (blockIdx.x / RB) << below;  // the node whose partials were formed
  const int e = (blockIdx.x % RB) * 256 + threadIdx.x;
  const Node nd = pddp_node(slot, p.level, p.Nq, p.G);
  if (nd.c <= 1 - below || e >= E) return;
  const int parts = (nd.n + p.cg - 1) / p.cg;
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
  if (below) p.red[(node + 1) * E + e] = p.red_prev[((size_t)bh * (1 << (p.level - 1)) + (slot >> 1)) * E + e] - s;
}

template <int D, bool BF16>
__global__ __launch_bounds__(kNodeThreads) void pddp_power_kernel(PddpParams p) {
  constexpr int E = kPartE<D, BF16>;
  __shared__ double sS[D], sR[D], sV[D];
  __shared__ double sX[kSymPart<D, BF16> ? 4 : 1][2][kSymPart<D, BF16> ? 1024 : 1];
  __shared__ __attribute__((aligned(16))) float sY[2][D];
  __shared__ double sMu[4];
  const int bh = blockIdx.y, slot = blockIdx.x;
  const Node nd = pddp_node(slot, p.level, p.Nq, p.G);
  if (nd.c <= 1) return;
  const size_t node = (size_t)bh * (1 << p.level) + slot;
  const double* red = p.red + node * E;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), ln = l & 31, h = l >> 5;
  double cacc[D / 32][16];
  if (tid < D) sS[tid] = red[tid];
  // the shift of the partial sums: the head's row 0 (bf16 inputs)
  const size_t hbase = (size_t)bh * p.Nq;
  if (BF16 && tid < D) sR[tid] = (double)(float)((const __bf16*)p.Q)[hbase * D + tid];
  if constexpr (BF16) store_mean<D>(p, bh, slot, sR, sS, nd.n);  // each thread its own entries
  if constexpr (kSymPart<D, BF16>) {
    // block (bi, W) of column W: stored as it is, or as the transpose of the
    // stored block (W, bi); element (r, c) of a stored block sits at
    // i*64 + l with r = 8*(i/4) + 4*(l/32) + i%4, c = l%32
    auto direct = [&](int bi, int m) {
#pragma unroll
      for (int i = 0; i < 16; ++i) cacc[bi][i] = red[D + m * 1024 + i * 64 + l];
    };
    // a transposed block passes through this wave's own LDS area (coalesced
    // global reads; element (r, c) at r*32 + (c ^ r), conflict-free both ways)
    auto transposed = [&](int bi, int m, int k) {
      double* X = sX[w][k];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * h + (i & 3);
        X[r * 32 + (ln ^ r)] = red[D + m * 1024 + i * 64 + l];
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // other lanes' stores before these reads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * h + (i & 3);
        cacc[bi][i] = X[ln * 32 + (r ^ ln)];
      }
    };
    switch (__builtin_amdgcn_readfirstlane(w)) {
      case 0: direct(0, 0); direct(1, 4); direct(2, 8); transposed(3, 7, 0); break;
      case 1: direct(1, 1); direct(2, 5); direct(3, 9); transposed(0, 4, 0); break;
      case 2: direct(2, 2); direct(3, 6); transposed(0, 8, 0); transposed(1, 5, 1); break;
      default: direct(3, 3); direct(0, 7); transposed(1, 9, 0); transposed(2, 6, 1); break;
    }
  } else if (w < D / 32) {
#pragma unroll
    for (int bi = 0; bi < D / 32; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        cacc[bi][i] = red[D + (size_t)(32 * bi + 8 * (i >> 2) + 4 * h + (i & 3)) * D + 32 * w + ln];
  }
  __syncthreads();
  // centred in fp64, iterated in fp32 (C rounded to fp32, as in the small-node
  // kernel): the steps' latency chain is half the fp64 one's
  const double inv_n = 1.0 / (double)nd.n;
  float cf[D / 32][16];
  if (w < D / 32) {
    const double sc = sS[w * 32 + ln] * inv_n;
#pragma unroll
    for (int bi = 0; bi < D / 32; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i) cf[bi][i] = (float)(cacc[bi][i] - sS[bi * 32 + 8 * (i >> 2) + 4 * h + (i & 3)] * sc);
  }
  power_f32<D>(cf, sY, sV, p.iters);
  const double mv = wave_sum_f64(tid < D ? ((BF16 ? sR[tid] : 0.0) + sS[tid] * inv_n) * sV[tid] : 0.0);
  if (l == 0 && w < 4) sMu[w] = mv;
  __syncthreads();
  const double muv = (sMu[0] + sMu[1]) + (sMu[2] + sMu[3]);
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
  size_t mean;            // bf16 values per level of node means
};

// Rows per partial scatter sum at a many-workgroup level (a multiple of 64,
// at least 512): the chunking whose rounds of two gram workgroups per CU
// (512 on 256 CUs) take the fewest tile times, each chunk's partial sums
// counted as 1/200 of a tile time (they are written and reduced).  (A fixed
// chunk of BH*Nq/512 rows gave every level a few more than 512 chunks, so
// each gram launch ran a second, almost empty round: twice its time; at 40
// heads one chunk per node left 320 long workgroups on 512 slots.)
constexpr int kGramSlots = 512;
long long gram_chunk_rows(long long maxn, int BH, int nslots) {
  const long long nodes = (long long)BH * nslots, tiles = (maxn + 63) / 64;
  long long best_rows = tiles * 64, best_cost = -1;
  for (long long c = 1; c <= tiles; ++c) {
    const long long rows = ((maxn + c - 1) / c + 63) / 64 * 64;
    if (rows < 512 && c > 1) break;
    const long long chunks = nodes * ((maxn + rows - 1) / rows);
    const long long rounds = (chunks + kGramSlots - 1) / kGramSlots;
    const long long cost = 200 * rounds * (rows / 64) + chunks;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_rows = rows;
    }
  }
  return best_rows;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Nodes per head whose scatter is summed at a many-workgroup level: the root,
// then the left child of each node (the right child's sums are derived).
int gram_nodes(int level) { return level > 0 ? 1 << (level - 1) : 1; }

long long level_max_rows(const Shape& s, int level) {
  const long long cmax = ((long long)s.c + (1LL << level) - 1) >> level;
  const long long n = cmax * s.G;
  return n < s.Nq ? n : s.Nq;
}

Plan make_plan(const Shape& s) {
  Plan pl{0, 0, 0, 0, 0, 0};
  while ((1 << pl.levels) < s.c) ++pl.levels;
  pl.mean = ((size_t)s.BH << (pl.levels > 0 ? pl.levels - 1 : 0)) * (size_t)s.d;
  long long cr = ((long long)s.BH * s.Nq + 511) / 512;
  cr = (cr + 63) / 64 * 64;
  pl.cr = (int)(cr < 1024 ? 1024 : (cr > kMaxChunkRows ? kMaxChunkRows : cr));
  const size_t E = (size_t)s.d + (size_t)s.d * s.d;
  for (int lv = 0; lv < pl.levels; ++lv) {
    const long long maxn = level_max_rows(s, lv);
    if (maxn <= pl.cr) break;
    const size_t nodes = (size_t)s.BH << lv;
    const long long cg = gram_chunk_rows(maxn, s.BH, gram_nodes(lv));
    const size_t pmax = (size_t)((maxn + cg - 1) / cg);
    pl.part = std::max(pl.part, nodes * pmax * E);
    pl.red = std::max(pl.red, nodes * E);
    pl.vec = std::max(pl.vec, nodes * ((size_t)s.d + 1));
  }
  return pl;
}

template <int D, bool BF16>
void launch_levels(const Shape& s, const Plan& pl, PddpParams p, hipStream_t st) {
  constexpr int RB = (kPartE<D, BF16> + 255) / 256;
  double* const red[2] = {p.red, p.red + pl.red};  // the level's sums and the level above's
  __bf16* const mean[2] = {p.mean_cur, p.mean_cur + pl.mean};
  for (int lv = 0; lv < pl.levels; ++lv) {
    p.level = lv;
    p.mean_cur = mean[lv & 1];
    p.mean_prev = mean[(lv + 1) & 1];
    const int nslots = 1 << lv;
    const long long maxn = level_max_rows(s, lv);
    if (maxn > pl.cr) {
      p.cg = (int)gram_chunk_rows(maxn, s.BH, gram_nodes(lv));
      p.pmax = (int)((maxn + p.cg - 1) / p.cg);
      p.red = red[lv & 1];
      p.red_prev = red[(lv + 1) & 1];
      const dim3 chunks(gram_nodes(lv) * p.pmax, s.BH);
      hipLaunchKernelGGL((pddp_gram_kernel<D, BF16>), chunks, dim3(kNodeThreads), 0, st, p);
      hipLaunchKernelGGL((pddp_reduce_kernel<D, BF16>), dim3(gram_nodes(lv) * RB, s.BH), dim3(256), 0, st, p);
      hipLaunchKernelGGL((pddp_power_kernel<D, BF16>), dim3(nslots, s.BH), dim3(kNodeThreads), 0, st, p);
      p.pj_pmax = (int)((maxn + kProjRows - 1) / kProjRows);
      hipLaunchKernelGGL((pddp_project_kernel<D, BF16>), dim3(nslots * p.pj_pmax, s.BH), dim3(256), 0, st, p);
      // the register cache sized to the node: the padding of a larger cache
      // reads as key 0 and all of it lands in one histogram bin of the
      // first radix pass (a 4096-row split in a 32768-key cache took as long
      // as a 32768-row one)
      // (1024 threads from 8193 keys on: the top levels run only a few of
      // these workgroups)
      if (maxn <= 8LL * kSplitThreads)
        hipLaunchKernelGGL((pddp_split_kernel<kSplitThreads, 8>), dim3(nslots, s.BH), dim3(kSplitThreads), 0, st, p);
      else if (maxn <= 16LL * kSplitThreads)
        hipLaunchKernelGGL((pddp_split_kernel<kSplitThreads, 16>), dim3(nslots, s.BH), dim3(kSplitThreads), 0, st, p);
      else if (maxn <= 16LL * kSplitWideThreads)
        hipLaunchKernelGGL((pddp_split_kernel<kSplitWideThreads, 16>), dim3(nslots, s.BH), dim3(kSplitWideThreads), 0,
                           st, p);
      else if (maxn <= 32LL * kSplitWideThreads)
        hipLaunchKernelGGL((pddp_split_kernel<kSplitWideThreads, 32>), dim3(nslots, s.BH), dim3(kSplitWideThreads), 0,
                           st, p);
      else if (maxn <= 80LL * kSplitWideThreads)
        hipLaunchKernelGGL((pddp_split_kernel<kSplitWideThreads, 80>), dim3(nslots, s.BH), dim3(kSplitWideThreads), 0,
                           st, p);
      else
        hipLaunchKernelGGL((pddp_split_kernel<kSplitWideThreads, 0>), dim3(nslots, s.BH), dim3(kSplitWideThreads), 0,
                           st, p);
    } else {
      const dim3 grid(nslots, s.BH);
      static_assert(kMaxChunkRows <= 16 * kNodeThreads, "node kernel register cache");
      if (BF16 && maxn <= kSmallRows)
        hipLaunchKernelGGL((pddp_small_kernel<D>), grid, dim3(kNodeThreads), 0, st, p);
      else if (maxn <= 2 * kNodeThreads)
        hipLaunchKernelGGL((pddp_node_kernel<D, BF16, 2>), grid, dim3(kNodeThreads), 0, st, p);
      else if (maxn <= 4 * kNodeThreads)
        hipLaunchKernelGGL((pddp_node_kernel<D, BF16, 4>), grid, dim3(kNodeThreads), 0, st, p);
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
  return 2 * round256(n * 4) + round256(pl.part * 8) + round256(2 * pl.red * 8) + round256(pl.vec * 8) +
         round256(2 * pl.mean * 2);
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
  w += round256(2 * pl.red * 8);
  p.vec = (double*)w;
  w += round256(pl.vec * 8);
  p.mean_cur = (__bf16*)w;
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
