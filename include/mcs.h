/*
 * mcs.h - MC-Sparse token-sparse attention for video diffusion transformers,
 * native on AMD Instinct MI355X (gfx950).
 *
 * Method: the review "[논문리뷰] MC-Sparse: Deconstructing and Closing the
 * Dense-Sparse Attention Gap in Diffusion Transformers" (blog.secrett2633.cloud),
 * section "3. Method & Key Results".  Queries are grouped into equal-size,
 * tile-aligned groups by Fast PDDP; at an anchor step exact attention is run,
 * each group keeps its top-k individual KV tokens by exact attention score, and
 * the residual R = O_full - O_sparse is stored; on the reuse steps that follow,
 * attention runs over the stored selections and R is added back.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Plain C ABI.  No exception crosses it.  Every call is asynchronous on the
 *    given HIP stream (a hipStream_t passed as void*; NULL = the default
 *    stream) and never synchronizes the host.
 *  - Every buffer is owned by the caller: device memory, contiguous, 16-byte
 *    aligned, not overlapping any other argument.  The library allocates
 *    nothing and keeps no state between calls; the cross-step state of the
 *    method (perm, idx, R) lives in caller buffers.
 *  - Layouts are row-major: Q [B,H,Nq,d], K and V [B,H,Nkv,d], O [B,H,Nq,d]
 *    (d fastest).  Tokens of a (frames x height x width) latent are flattened
 *    frame-major, n = (t*height + y)*width + x.
 *  - Q, K, V and O have element type `dtype`; the residual R is float32
 *    unless `r_dtype` asks for bf16; lse and scores are float32.
 *  - Query row i sits at position q_offset + i of the KV sequence.  With
 *    causal_block == 0 every key is visible; otherwise key j is visible to
 *    query i iff j / causal_block <= (q_offset + i) / causal_block
 *    (frame-block causal attention for chunked video generation).
 *  - Errors: argument checks run on the host before anything is enqueued and
 *    leave every output untouched; a failed launch returns MCS_ERR_HIP.
 *    mcs_last_error() gives a human-readable detail (thread-local).
 *    Numerical problems (NaN/Inf inputs) are not detected.
 *  - Calls that share a workspace or output buffer must not overlap in time.
 */
#ifndef MCS_H_
#define MCS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mcs_status {
  MCS_OK = 0,
  MCS_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or parameter  */
  MCS_ERR_UNSUPPORTED = 2, /* valid but not implemented (d, G or dtype)       */
  MCS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
  MCS_ERR_HIP = 4          /* HIP runtime error while enqueueing              */
} mcs_status;

typedef enum mcs_dtype { MCS_F32 = 0, MCS_BF16 = 1 } mcs_dtype;

/* How mcs_anchor forms the selections; both give the same idx bit for bit. */
typedef enum mcs_anchor_mode {
  MCS_ANCHOR_AUTO = 0,        /* the library chooses (default)                           */
  MCS_ANCHOR_TWO_PASS = 1,    /* column-mass matrix in the workspace, then a top-k pass   */
  MCS_ANCHOR_SINGLE_PASS = 2  /* each group's mass kept on chip and selected in the same  */
                              /* workgroup; bf16 only, visible keys of the chunk <= 32768 */
} mcs_anchor_mode;

typedef enum mcs_workspace_kind {
  MCS_WS_GROUP = 0,
  MCS_WS_ANCHOR = 1,
  MCS_WS_BLOCK = 2,
  MCS_WS_DRIFT = 3
} mcs_workspace_kind;

/* Problem description.  Supported: d in {64,128}; group_size in {64,128};
 * 1 <= k <= Nkv; Nq, Nkv <= 2^24; Nkv*d*4 < 2^31 (one head's K or V is
 * addressed with 32-bit byte offsets); B*H*max(Nq,Nkv)*d < 2^40; r_dtype
 * MCS_BF16 only with dtype MCS_BF16.  Others return MCS_ERR_UNSUPPORTED or
 * MCS_ERR_INVALID_ARG before any launch.  A zero-initialised struct with the
 * sizes filled in selects the defaults (float32 data and residual). */
typedef struct mcs_problem {
  int32_t B, H;         /* batch, heads                                        */
  int32_t Nq, Nkv;      /* query and key/value tokens per head (Nq may be 0)   */
  int32_t d;            /* head dimension                                      */
  int32_t group_size;   /* G: queries per group; groups c = ceil(Nq/G), only   */
                        /* the last group (depth-first order) may be short     */
  int32_t k;            /* KV tokens kept per group                            */
  float scale;          /* logit multiplier (usually 1/sqrt(d)); finite, > 0   */
  int32_t causal_block; /* 0: bidirectional; else tokens per causal block      */
  int32_t q_offset;     /* position of query 0 in the KV sequence (>= 0)      */
  int32_t pddp_iters;   /* power-iteration steps per PDDP split (0..1024)      */
  int32_t dtype;        /* mcs_dtype of Q, K, V, O                             */
  int32_t r_dtype;      /* mcs_dtype of the residual R: MCS_F32 (0, default),  */
                        /* the difference of the float32 outputs stored whole; */
                        /* MCS_BF16 (bf16 problems only) rounds it once more   */
                        /* and halves its bytes                                */
  int32_t anchor_mode;  /* mcs_anchor_mode (0: automatic)                      */
} mcs_problem;

/* Bytes of workspace mcs_group (kind MCS_WS_GROUP), mcs_anchor
 * (MCS_WS_ANCHOR), mcs_block_select (MCS_WS_BLOCK) or mcs_residual_drift
 * (MCS_WS_DRIFT, sized for its largest n_rows) needs to process all B*H heads
 * in one pass.  For
 * MCS_WS_ANCHOR any size of at least `*min_bytes` works (heads are then
 * processed in chunks); min_bytes may be NULL.  For bf16 problems the anchor
 * workspace also holds the float32 O_full of all heads (B*H*Nq*d*4 bytes, part
 * of the minimum).  Pure host computation. */
mcs_status mcs_workspace_size(const mcs_problem* p, int32_t kind, size_t* bytes, size_t* min_bytes);

/* Fast-PDDP query grouping (MC-Sparse review, section 3: equal-size,
 * tile-aligned groups of similar queries).  Per (b,h), the queries are split
 * recursively: a node holding c >= 2 groups is centred on its mean, its scatter
 * matrix C = Xc^T Xc is formed, the direction v = C^T v0 / ||C^T v0||
 * (v0 = all-ones / sqrt(d), T = pddp_iters steps, each normalised; a zero
 * product keeps the previous direction) is computed, the projections
 * p = Xc v are ranked by (p, original index), and the first floor(c/2)*G
 * ranked queries form the left child.  Groups are numbered depth-first
 * (left first).
 *   Q    [B,H,Nq,d] dtype, read only.
 *   perm [B,H,Nq] int32, written: perm[b,h,g*G + r] is the r-th member of
 *        group g, members ascending within a group.
 *   ws   workspace of at least mcs_workspace_size(MCS_WS_GROUP) bytes. */
mcs_status mcs_group(const mcs_problem* p, const void* Q, int32_t* perm, void* ws, size_t ws_bytes,
                     void* stream);

/* Exact (dense) softmax attention over all 3D tokens, whose quadratic cost
 * is the bottleneck the method removes (MC-Sparse review, section 2
 * "Motivation"; FrameDiT summary, gist.science, "1. 연구 배경"), the output
 * MC-Sparse approximates and the speed comparator:
 * O_i = sum_j softmax_j(scale * <q_i, k_j>) v_j over the visible keys.
 *   O   [B,H,Nq,d] dtype, written.
 *   lse [B,H,Nq] float32 or NULL: natural-log normaliser log sum_j exp(...)
 *       of each row (-inf for a row with no visible key, whose O is 0). */
mcs_status mcs_dense_attn(const mcs_problem* p, const void* Q, const void* K, const void* V, void* O,
                          float* lse, void* stream);

/* Anchor step (MC-Sparse review, section 3: exact scores at the anchor,
 * token-level selection, residual compensation).  Given the groups `perm`
 * (from mcs_group on this step's Q), it runs exact attention, computes for
 * each group g the exact attention mass every key receives,
 *   m_g[j] = sum_{i in g} exp(scale*<q_i,k_j> - lse_i)   (0 if not visible),
 * keeps the k keys with the largest mass (ties to the lower index; with
 * anchor_mode MCS_ANCHOR_SINGLE_PASS each group's masses stay on chip and are
 * selected in the same pass, see mcs_anchor_mode), runs
 * attention restricted to those keys (softmax renormalised over the selected
 * keys visible to each query; a query with none gets 0) and stores the
 * residual R = O_full - O_sparse.
 *   perm [B,H,Nq] int32, read (a valid grouping; not checked on the device).
 *   O    [B,H,Nq,d] dtype, written with O_full (rounded to dtype).
 *   idx  [B,H,c,k] int32, written: each group's selected key indices, ascending.
 *   R    [B,H,Nq,d] r_dtype, written (original token order): O_full - O_sparse
 *        formed in float32 from the unrounded O_full (float32 by default;
 *        rounded once to bf16 when r_dtype is MCS_BF16).
 *   ws   workspace of at least the minimum mcs_workspace_size(MCS_WS_ANCHOR). */
mcs_status mcs_anchor(const mcs_problem* p, const void* Q, const void* K, const void* V,
                      const int32_t* perm, void* O, int32_t* idx, void* R, void* ws, size_t ws_bytes,
                      void* stream);

/* Reuse step (MC-Sparse review, section 3): gathered sparse attention of each
 * group's queries over that group's stored selection, on the current step's
 * Q/K/V, plus the stored residual as an additive correction:
 *   O_i = sum_{j in S_g(i), visible} softmax_j(scale*<q_i,k_j>) v_j + R_i.
 *   perm, idx from the anchor (perm must be a permutation of [0,Nq) and idx
 *   values in [0,Nkv); not checked on the device).
 *   R    [B,H,Nq,d] r_dtype from the anchor, or NULL for plain sparse
 *        attention; added in float32, the sum rounded once to dtype.
 *   O    [B,H,Nq,d] dtype, written (may not alias Q, K, V or R). */
mcs_status mcs_sparse_attn(const mcs_problem* p, const void* Q, const void* K, const void* V,
                           const int32_t* perm, const int32_t* idx, const void* R, void* O,
                           void* stream);

/* Selection of the block-sparse comparator, recomputed on every step
 * (MC-Sparse review, section 1: selection error of approximate scoring such as
 * mean pooling, structural binding error of whole-block selection; section 2:
 * block-sparse attention).  Query blocks are the G-token tiles of the token
 * order and KV blocks the 64-token tiles (each last tile may be short).  With
 * mean pooled block vectors, KV block b scores scale*<mean q_g, mean k_b> for
 * query block g; blocks with no key visible to any query of g rank last.
 * Blocks are taken by decreasing score (ties to the lower block index) while
 * the token count stays within k, and the next block gives its lowest-index
 * tokens up to exactly k.  The outputs have the shapes mcs_anchor gives, so
 * mcs_sparse_attn(perm, idx, R = NULL) then runs the block-sparse attention.
 *   perm [B,H,Nq] int32, written with the identity (query blocks are tiles).
 *   idx  [B,H,c,k] int32, written: each query block's selected tokens, ascending.
 *   ws   workspace of at least mcs_workspace_size(MCS_WS_BLOCK) bytes
 *        (float32 pooled vectors of every tile).
 * Unsupported (MCS_ERR_UNSUPPORTED): more than 8192 KV blocks (Nkv > 524288)
 * or k > 32705 (more than 512 blocks to rank). */
mcs_status mcs_block_select(const mcs_problem* p, const void* Q, const void* K, int32_t* perm, int32_t* idx,
                            void* ws, size_t ws_bytes, void* stream);

/* Residual-drift check for adaptive anchoring (MC-Sparse review, section 3:
 * selections and the dense-sparse residual are reused because they are
 * temporally stable; this measures how far they have moved).  For every head
 * the sampled query rows get exact attention in float32 (split over key
 * ranges), and
 *   drift[b,h] = ||O[rows] - O_exact[rows]||_F / ||O_exact[rows]||_F
 * (0 when O_exact is 0 on every sampled row), O being the caller's output for
 * this step.  For a reuse output O = O_sparse + R_anchor this is the movement
 * of the residual since the anchor, R_anchor - R_now, relative to the output;
 * a caller anchors again when it exceeds a threshold.
 *   O      [B,H,Nq,d] dtype, read (the step's output, e.g. from mcs_sparse_attn).
 *   rows   [n_rows] int32 device memory: token indices in [0,Nq), the same
 *          for every head (clamped into range on the device).
 *   n_rows 1..128.
 *   drift  [B*H + 1] float32 device memory, written: drift[b*H + h] for each
 *          head, then drift[B*H] = the largest of them (NaN if any is NaN),
 *          the value an anchor schedule compares with its threshold.
 *   ws     workspace of at least mcs_workspace_size(MCS_WS_DRIFT) bytes. */
mcs_status mcs_residual_drift(const mcs_problem* p, const void* Q, const void* K, const void* V, const void* O,
                              const int32_t* rows, int32_t n_rows, float* drift, void* ws, size_t ws_bytes,
                              void* stream);

/* mcs_residual_drift without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and results as
 * mcs_residual_drift; its scratch is a static device array of 64 MiB (one
 * copy per GPU, held until the process ends), whose address on the current
 * device is looked up on the first call there.  The call allocates nothing.
 *   Scratch needed: 4*B*H*n_rows*(nsplit*(d + 2) + 2) bytes with nsplit =
 *   ceil(ceil(Nkv/64) / max(8, ceil(ceil(Nkv/64)/64))) key ranges (at most
 *   64); a problem needing more than 64 MiB returns MCS_ERR_WORKSPACE before
 *   any launch (32760 keys, 12 heads, d = 128 fit all 128 rows; 75600 keys,
 *   40 heads, d = 128 up to 51).
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (other streams or threads) race and must be serialised by the
 *   caller.  Nothing needs clearing between calls: every scratch value a
 *   call reads is first written by that call. */
mcs_status mcs_residual_drift_noalloc(const mcs_problem* p, const void* Q, const void* K, const void* V,
                                      const void* O, const int32_t* rows, int32_t n_rows, float* drift,
                                      void* stream);

/* Static description of a status code. */
const char* mcs_status_string(mcs_status s);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char* mcs_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int32_t mcs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MCS_H_ */
