// Token-level top-k selection per query group (MC-Sparse review,
// blog.secrett2633.cloud, section 3: each group keeps the individual KV
// tokens of largest exact attention mass).
//
// One 512-thread workgroup per group row of the mass matrix.  The masses are
// non-negative floats, so their bit patterns order like the values (a -0 is
// read as +0).  The block select (select.hpp) finds the k-th largest pattern
// and emits the kept keys in ascending index order, equal masses taken
// lowest index first.  The patterns of non-negative floats are below 2^31, so
// the first radix pass takes bits 30..19 (8 exponent and 4 mantissa bits):
// twice the bins of a pass over bits 31..20, half the atomic contention on
// rows whose masses share few octaves.  Rows of up to 81920 keys are held in
// registers (up to 64 keys per thread of a 512-thread workgroup, or 80 of a
// 1024-thread one; one HBM read); longer rows are re-read on each pass,
// sixteen keys per thread in flight.
#include "mcs_kernels.hpp"
#include "select.hpp"

namespace mcs {
namespace {

constexpr int kTopkThreads = 512;
constexpr int kTopkWideThreads = 1024;  // rows of 32769..81920 keys: 80 per thread

struct TopkParams {
  const float* mass;
  int32_t* idx;
  int Nkv, k, c, bh0;
};

struct MassKeys {
  const uint32_t* row;
  __device__ __forceinline__ uint32_t operator()(int j) const {
    const uint32_t u = row[j];
    return (u & 0x80000000u) ? 0u : u;
  }
};

template <int NT, int VPT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkParams p) {
  using Sel = BlockSelect<NT, VPT>;
  __shared__ typename Sel::Shared sh;
  const int unit = blockIdx.x;
  const int bhl = unit / p.c, g = unit - bhl * p.c;
  const MassKeys keys{(const uint32_t*)(p.mass + (size_t)unit * p.Nkv)};
  int32_t* out = p.idx + ((size_t)(p.bh0 + bhl) * p.c + g) * p.k;
  Sel sel;
  sel.n = p.Nkv;
  sel.load(keys);
  uint32_t T;
  int tie_need;
  sel.template threshold<31>(keys, p.k, sh, T, tie_need);
  sel.split(keys, T, tie_need, sh, [&](int, int j, bool s, int pos) {
    if (s && pos < p.k) out[pos] = j;  // pos < k by construction; checked so that no error can write past the row
  });
}

template <int NT, int VPT>
void launch(const TopkParams& p, int rows, hipStream_t st) {
  hipLaunchKernelGGL((topk_kernel<NT, VPT>), dim3(rows), dim3(NT), 0, st, p);
}

}  // namespace

hipError_t launch_topk(const Shape& s, int bh0, int nbh, const float* mass, int32_t* idx, hipStream_t st) {
  const TopkParams p{mass, idx, s.Nkv, s.k, s.c, bh0};
  const int rows = nbh * s.c;
  if (s.Nkv <= 4 * kTopkThreads) launch<kTopkThreads, 4>(p, rows, st);
  else if (s.Nkv <= 16 * kTopkThreads) launch<kTopkThreads, 16>(p, rows, st);
  else if (s.Nkv <= 64 * kTopkThreads) launch<kTopkThreads, 64>(p, rows, st);
  else if (s.Nkv <= 80 * kTopkWideThreads) launch<kTopkWideThreads, 80>(p, rows, st);
  else launch<kTopkThreads, 0>(p, rows, st);
  return hipGetLastError();
}

}  // namespace mcs
