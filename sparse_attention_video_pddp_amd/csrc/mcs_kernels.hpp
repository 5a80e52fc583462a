// Internal launch interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcs {

// Validated problem, flattened for the launchers.
struct Shape {
  int BH;        // B * H
  int Nq, Nkv, d;
  int G, k, c;   // group size, kept keys, groups per head
  float scale;
  int causal_block, q_offset, iters;
};

// Dense attention (exact).  O in dtype; lse (natural log) and Ofull (fp32
// copy of the unrounded output) are optional.
hipError_t launch_dense_bf16(const Shape& s, const void* Q, const void* K, const void* V, void* O,
                             float* lse, float* Ofull, hipStream_t st);
hipError_t launch_dense_f32(const Shape& s, const void* Q, const void* K, const void* V, void* O,
                            float* lse, float* Ofull, hipStream_t st);

// Per-group exact column mass for heads [bh0, bh0 + nbh): mass[(bh-bh0)*c + g][Nkv].
hipError_t launch_mass_bf16(const Shape& s, int bh0, int nbh, const void* Q, const void* K,
                            const int32_t* perm, const float* lse, float* mass, hipStream_t st);
hipError_t launch_mass_f32(const Shape& s, int bh0, int nbh, const void* Q, const void* K,
                           const int32_t* perm, const float* lse, float* mass, hipStream_t st);

// Single-pass anchor selection (bf16): per group, the column mass over the
// launch's visible keys [0, fused_anchor_row(s)) kept in LDS and its top-k
// selected in the same workgroup; idx equals the two-pass path's.  Rows of
// at most kFusedMaxKv keys.
constexpr int kFusedMaxKv = 32768;
int fused_anchor_row(const Shape& s);
hipError_t launch_anchor_fused_bf16(const Shape& s, const void* Q, const void* K, const int32_t* perm,
                                    const float* lse, int32_t* idx, hipStream_t st);

// Top-k per group row of `mass` (heads [bh0, bh0+nbh)), written to idx[bh][g][k] ascending.
hipError_t launch_topk(const Shape& s, int bh0, int nbh, const float* mass, int32_t* idx, hipStream_t st);

// Gathered sparse attention, bf16 inputs.  anchor: R <- Ofull - O_sparse
// (Ofull: the float32 dense output), stored as float32 (r_f32) or rounded to
// bf16.  reuse: O <- O_sparse + R (R may be null).
hipError_t launch_sparse_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                              const int32_t* perm, const int32_t* idx, const float* Ofull, void* R, bool r_f32,
                              void* O, bool anchor, hipStream_t st);
// float32: anchor: R <- R - O_sparse (R holds O_full on entry); reuse as above.
hipError_t launch_sparse_f32(const Shape& s, const void* Q, const void* K, const void* V,
                             const int32_t* perm, const int32_t* idx, float* R, void* O, bool anchor,
                             hipStream_t st);

// Block-sparse comparator (mean-pooled block selection).  KV blocks of
// kPoolBlock tokens; the scores of one query block's KV blocks are held in
// LDS (at most kMaxKvBlocks) and the top J of them are ranked exactly (at
// most kMaxSelBlocks).
constexpr int kPoolBlock = 64;
constexpr int kMaxKvBlocks = 8192;
constexpr int kMaxSelBlocks = 512;
// Blocks that certainly hold k tokens: J-1 full blocks and at least one more
// token (every block but the last has kPoolBlock tokens).
inline __host__ __device__ int block_select_count(int k, int nkb) {
  const int j = (k - 1 + kPoolBlock - 1) / kPoolBlock + 1;
  return j < nkb ? j : nkb;
}
// ws: float32 pooled queries [BH][c][d] then pooled keys [BH][d][nkb].
size_t block_workspace_bytes(const Shape& s);
hipError_t launch_block_select(const Shape& s, bool bf16, const void* Q, const void* K, int32_t* perm,
                               int32_t* idx, void* ws, hipStream_t st);

// Residual-drift check: exact attention of at most kMaxDriftRows sampled
// query rows per head, split over at most kMaxDriftSplits key ranges;
// drift[BH] receives the largest per-head value.
constexpr int kMaxDriftRows = 128;
constexpr int kMaxDriftSplits = 64;
// Scratch of a check over n_rows sampled rows (every value read is first
// written by the same call: nothing needs clearing).
size_t drift_workspace_bytes(const Shape& s, int n_rows);
hipError_t launch_drift(const Shape& s, bool bf16, const void* Q, const void* K, const void* V, const void* O,
                        const int32_t* rows, int n_rows, float* drift, void* ws, hipStream_t st);

// PDDP grouping.  ws: int32 tmp [BH*Nq] followed by uint32 keys [BH*Nq].
size_t pddp_workspace_bytes(const Shape& s);
hipError_t launch_pddp(const Shape& s, bool bf16, const void* Q, int32_t* perm, void* ws, hipStream_t st);

}  // namespace mcs
