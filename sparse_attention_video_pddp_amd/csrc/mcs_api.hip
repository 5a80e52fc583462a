// C ABI of the library (declared in include/mcs.h): argument validation on
// the host before anything is enqueued, workspace sizing, kernel dispatch.
// Stateless: every buffer is the caller's, nothing is allocated here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "mcs.h"
#include "mcs_kernels.hpp"

namespace {

thread_local std::string g_last_error;

mcs_status fail(mcs_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mcs_status ok() {
  g_last_error.clear();
  return MCS_OK;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Checked {
  mcs::Shape s;
  bool bf16;
  bool r_f32;        // the residual is float32
  bool single_pass;  // mcs_anchor keeps each group's mass on chip (mcs_anchor_mode)
  bool empty;
};

// The automatic anchor mode takes the single pass for rows of visible keys up
// to this length.  Measured on the frame-causal video (4680 queries, 12
// heads, d = 128, group + anchor per chunk): 4680 visible keys 0.81 ms single
// against 0.99 ms two-pass, 9360 keys 1.08 against 1.12, 14040 keys 1.36
// against 1.27, 32760 keys 2.65 against 1.99; the single pass re-reads the
// visible K rows for every group, the two-pass path writes and re-reads the
// mass matrix and launches twice.
constexpr int kSinglePassAutoKv = 12288;

// Pure host checks of the problem description.
mcs_status check_problem(const mcs_problem* p, Checked& out) {
  if (!p) return fail(MCS_ERR_INVALID_ARG, "problem is NULL");
  if (p->B < 0 || p->H < 0) return fail(MCS_ERR_INVALID_ARG, "B=%d H=%d must be >= 0", p->B, p->H);
  if ((long long)p->B * p->H > 65535)
    return fail(MCS_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)p->B * p->H);
  if (p->Nq < 0 || p->Nq > (1 << 24)) return fail(MCS_ERR_INVALID_ARG, "Nq=%d outside [0, 2^24]", p->Nq);
  if (p->Nkv < 1 || p->Nkv > (1 << 24)) return fail(MCS_ERR_INVALID_ARG, "Nkv=%d outside [1, 2^24]", p->Nkv);
  if (p->d != 64 && p->d != 128) return fail(MCS_ERR_UNSUPPORTED, "d=%d (supported: 64, 128)", p->d);
  if (p->group_size != 64 && p->group_size != 128)
    return fail(MCS_ERR_UNSUPPORTED, "group_size=%d (supported: 64, 128)", p->group_size);
  if (p->k < 1 || p->k > p->Nkv) return fail(MCS_ERR_INVALID_ARG, "k=%d outside [1, Nkv=%d]", p->k, p->Nkv);
  if (!std::isfinite(p->scale) || !(p->scale > 0.f))
    return fail(MCS_ERR_INVALID_ARG, "scale=%g must be finite and > 0", (double)p->scale);
  if (p->causal_block < 0) return fail(MCS_ERR_INVALID_ARG, "causal_block=%d < 0", p->causal_block);
  if (p->q_offset < 0 || p->q_offset > (1 << 30))
    return fail(MCS_ERR_INVALID_ARG, "q_offset=%d outside [0, 2^30]", p->q_offset);
  if (p->pddp_iters < 0 || p->pddp_iters > 1024)
    return fail(MCS_ERR_INVALID_ARG, "pddp_iters=%d outside [0, 1024]", p->pddp_iters);
  if (p->dtype != MCS_F32 && p->dtype != MCS_BF16) return fail(MCS_ERR_UNSUPPORTED, "dtype=%d", p->dtype);
  const long long bh = (long long)p->B * p->H;
  const long long nmax = p->Nq > p->Nkv ? p->Nq : p->Nkv;
  if (bh * nmax * p->d >= (1LL << 40)) return fail(MCS_ERR_UNSUPPORTED, "tensor sizes exceed 2^40 elements");
  if (p->r_dtype != MCS_F32 && p->r_dtype != MCS_BF16) return fail(MCS_ERR_UNSUPPORTED, "r_dtype=%d", p->r_dtype);
  if (p->r_dtype == MCS_BF16 && p->dtype != MCS_BF16)
    return fail(MCS_ERR_UNSUPPORTED, "a bf16 residual needs bf16 inputs (dtype=%d)", p->dtype);
  if (p->anchor_mode < MCS_ANCHOR_AUTO || p->anchor_mode > MCS_ANCHOR_SINGLE_PASS)
    return fail(MCS_ERR_INVALID_ARG, "anchor_mode=%d", p->anchor_mode);
  // K and V rows of one head are addressed with 32-bit byte offsets (buffer loads)
  if ((long long)p->Nkv * p->d * 4 > 0x7fffffffLL)
    return fail(MCS_ERR_UNSUPPORTED, "Nkv=%d: one head's K or V exceeds 2^31 bytes", p->Nkv);
  const int c = (p->Nq + p->group_size - 1) / p->group_size;
  out.s = mcs::Shape{(int)bh,  p->Nq, p->Nkv, p->d, p->group_size, p->k, c, p->scale, p->causal_block,
                     p->q_offset, p->pddp_iters};
  out.bf16 = p->dtype == MCS_BF16;
  out.r_f32 = p->r_dtype == MCS_F32;
  out.empty = bh == 0 || p->Nq == 0;
  out.single_pass = false;
  if (!out.empty) {
    const int row = mcs::fused_anchor_row(out.s);
    const bool fits = out.bf16 && row <= mcs::kFusedMaxKv;
    if (p->anchor_mode == MCS_ANCHOR_SINGLE_PASS && !fits)
      return fail(MCS_ERR_UNSUPPORTED, "single-pass anchor needs bf16 inputs and at most %d visible keys (%d)",
                  mcs::kFusedMaxKv, row);
    out.single_pass = p->anchor_mode == MCS_ANCHOR_SINGLE_PASS ||
                      (p->anchor_mode == MCS_ANCHOR_AUTO && fits && row <= kSinglePassAutoKv);
  }
  return MCS_OK;
}

mcs_status check_host_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(MCS_ERR_INVALID_ARG, "%s is NULL", name);
  if ((uintptr_t)ptr % 16) return fail(MCS_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MCS_OK;
}

// Device-residency check (a HIP runtime query, no GPU work).
mcs_status check_dev_ptr(const void* ptr, const char* name) {
  hipPointerAttribute_t a;
  const hipError_t e = hipPointerGetAttributes(&a, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MCS_ERR_INVALID_ARG, "%s is not device memory (%s)", name, hipGetErrorString(e));
  }
  if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged)
    return fail(MCS_ERR_INVALID_ARG, "%s is not device memory", name);
  return MCS_OK;
}

struct Ptr {
  const void* p;
  const char* name;
  bool optional;
};

mcs_status check_ptrs(std::initializer_list<Ptr> ptrs) {
  for (const Ptr& x : ptrs) {
    if (x.optional && !x.p) continue;
    if (mcs_status s = check_host_ptr(x.p, x.name)) return s;
  }
  for (const Ptr& x : ptrs) {
    if (x.optional && !x.p) continue;
    if (mcs_status s = check_dev_ptr(x.p, x.name)) return s;
  }
  return MCS_OK;
}

size_t anchor_lse_bytes(const mcs::Shape& s) { return round_up((size_t)s.BH * s.Nq * 4); }
// bf16: the float32 dense output of all heads, kept until the residual is formed
size_t anchor_ofull_bytes(const mcs::Shape& s, bool bf16) {
  return bf16 ? round_up((size_t)s.BH * s.Nq * s.d * 4) : 0;
}
size_t anchor_mass_bytes_per_head(const mcs::Shape& s) { return round_up((size_t)s.c * s.Nkv * 4); }
// mass matrix bytes of the anchor: none for the single pass
size_t anchor_mass_bytes(const Checked& c) { return c.single_pass ? 0 : anchor_mass_bytes_per_head(c.s); }

mcs_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MCS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Scratch of mcs_residual_drift_noalloc: a fixed array in device memory, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in): its device address on the current GPU is looked up once with
// hipGetSymbolAddress and kept per device.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

mcs_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MCS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MCS_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MCS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MCS_OK;
}

}  // namespace

extern "C" {

const char* mcs_status_string(mcs_status s) {
  switch (s) {
    case MCS_OK: return "MCS_OK";
    case MCS_ERR_INVALID_ARG: return "MCS_ERR_INVALID_ARG";
    case MCS_ERR_UNSUPPORTED: return "MCS_ERR_UNSUPPORTED";
    case MCS_ERR_WORKSPACE: return "MCS_ERR_WORKSPACE";
    case MCS_ERR_HIP: return "MCS_ERR_HIP";
  }
  return "MCS_ERR_UNKNOWN";
}

const char* mcs_last_error(void) { return g_last_error.c_str(); }

int32_t mcs_version(void) { return 100; }

mcs_status mcs_workspace_size(const mcs_problem* p, int32_t kind, size_t* bytes, size_t* min_bytes) {
  Checked c;
  if (mcs_status s = check_problem(p, c)) return s;
  if (!bytes) return fail(MCS_ERR_INVALID_ARG, "bytes is NULL");
  size_t need = 0, need_min = 0;
  if (kind == MCS_WS_GROUP) {
    need = need_min = c.empty ? 0 : mcs::pddp_workspace_bytes(c.s);
  } else if (kind == MCS_WS_ANCHOR) {
    if (!c.empty) {
      const size_t fixed = anchor_lse_bytes(c.s) + anchor_ofull_bytes(c.s, c.bf16);
      need = fixed + (size_t)c.s.BH * anchor_mass_bytes(c);
      need_min = fixed + anchor_mass_bytes(c);
    }
  } else if (kind == MCS_WS_BLOCK) {
    need = need_min = c.empty ? 0 : mcs::block_workspace_bytes(c.s);
  } else if (kind == MCS_WS_DRIFT) {
    need = need_min = c.empty ? 0 : mcs::drift_workspace_bytes(c.s, mcs::kMaxDriftRows);
  } else {
    return fail(MCS_ERR_INVALID_ARG, "unknown workspace kind %d", kind);
  }
  *bytes = need;
  if (min_bytes) *min_bytes = need_min;
  return ok();
}

mcs_status mcs_group(const mcs_problem* p, const void* Q, int32_t* perm, void* ws, size_t ws_bytes,
                     void* stream) {
  Checked c;
  if (mcs_status s = check_problem(p, c)) return s;
  if (c.empty) return ok();
  const size_t need = mcs::pddp_workspace_bytes(c.s);
  if (mcs_status s = check_ptrs({{Q, "Q", false}, {perm, "perm", false}, {ws, "ws", false}})) return s;
  if (ws_bytes < need) return fail(MCS_ERR_WORKSPACE, "group workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(mcs::launch_pddp(c.s, c.bf16, Q, perm, ws, (hipStream_t)stream), "mcs_group");
}

mcs_status mcs_dense_attn(const mcs_problem* p, const void* Q, const void* K, const void* V, void* O,
                          float* lse, void* stream) {
  Checked c;
  if (mcs_status s = check_problem(p, c)) return s;
  if (c.empty) return ok();
  if (mcs_status s = check_ptrs({{Q, "Q", false}, {K, "K", false}, {V, "V", false}, {O, "O", false},
                                 {lse, "lse", true}}))
    return s;
  if (O == Q || O == K || O == V) return fail(MCS_ERR_INVALID_ARG, "O aliases an input");
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = c.bf16 ? mcs::launch_dense_bf16(c.s, Q, K, V, O, lse, nullptr, st)
                              : mcs::launch_dense_f32(c.s, Q, K, V, O, lse, nullptr, st);
  return hip_status(e, "mcs_dense_attn");
}

mcs_status mcs_anchor(const mcs_problem* p, const void* Q, const void* K, const void* V,
                      const int32_t* perm, void* O, int32_t* idx, void* R, void* ws, size_t ws_bytes,
                      void* stream) {
  Checked c;
  if (mcs_status s = check_problem(p, c)) return s;
  if (c.empty) return ok();
  if (mcs_status s = check_ptrs({{Q, "Q", false}, {K, "K", false}, {V, "V", false}, {perm, "perm", false},
                                 {O, "O", false}, {idx, "idx", false}, {R, "R", false}, {ws, "ws", false}}))
    return s;
  if (O == Q || O == K || O == V || R == O || R == Q || R == K || R == V)
    return fail(MCS_ERR_INVALID_ARG, "an output aliases another argument");
  const size_t lse_b = anchor_lse_bytes(c.s), of_b = anchor_ofull_bytes(c.s, c.bf16);
  const size_t head_b = anchor_mass_bytes(c);
  if (ws_bytes < lse_b + of_b + head_b)
    return fail(MCS_ERR_WORKSPACE, "anchor workspace %zu < minimum %zu bytes", ws_bytes, lse_b + of_b + head_b);
  const size_t fit = head_b ? (ws_bytes - lse_b - of_b) / head_b : (size_t)c.s.BH;
  const int chunk = fit >= (size_t)c.s.BH ? c.s.BH : (int)fit;
  float* lse = (float*)ws;
  // bf16: O_full (float32) in the workspace; float32: straight into R
  float* ofull = c.bf16 ? (float*)((char*)ws + lse_b) : (float*)R;
  float* mass = (float*)((char*)ws + lse_b + of_b);
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e = c.bf16 ? mcs::launch_dense_bf16(c.s, Q, K, V, O, lse, ofull, st)
                        : mcs::launch_dense_f32(c.s, Q, K, V, O, lse, ofull, st);
  if (e != hipSuccess) return hip_status(e, "mcs_anchor (dense)");
  if (c.single_pass) {
    e = mcs::launch_anchor_fused_bf16(c.s, Q, K, perm, lse, idx, st);
    if (e != hipSuccess) return hip_status(e, "mcs_anchor (single-pass selection)");
  }
  for (int bh0 = 0; !c.single_pass && bh0 < c.s.BH; bh0 += chunk) {
    const int nbh = c.s.BH - bh0 < chunk ? c.s.BH - bh0 : chunk;
    e = c.bf16 ? mcs::launch_mass_bf16(c.s, bh0, nbh, Q, K, perm, lse, mass, st)
               : mcs::launch_mass_f32(c.s, bh0, nbh, Q, K, perm, lse, mass, st);
    if (e != hipSuccess) return hip_status(e, "mcs_anchor (mass)");
    e = mcs::launch_topk(c.s, bh0, nbh, mass, idx, st);
    if (e != hipSuccess) return hip_status(e, "mcs_anchor (top-k)");
  }
  e = c.bf16 ? mcs::launch_sparse_bf16(c.s, Q, K, V, perm, idx, ofull, R, c.r_f32, nullptr, true, st)
             : mcs::launch_sparse_f32(c.s, Q, K, V, perm, idx, (float*)R, nullptr, true, st);
  return hip_status(e, "mcs_anchor (sparse)");
}

mcs_status mcs_block_select(const mcs_problem* p, const void* Q, const void* K, int32_t* perm, int32_t* idx,
                            void* ws, size_t ws_bytes, void* stream) {
  Checked c;
  if (mcs_status s = check_problem(p, c)) return s;
  const int nkb = (p->Nkv + mcs::kPoolBlock - 1) / mcs::kPoolBlock;
  if (nkb > mcs::kMaxKvBlocks)
    return fail(MCS_ERR_UNSUPPORTED, "Nkv=%d: %d KV blocks exceed %d", p->Nkv, nkb, mcs::kMaxKvBlocks);
  if (mcs::block_select_count(p->k, nkb) > mcs::kMaxSelBlocks)
    return fail(MCS_ERR_UNSUPPORTED, "k=%d needs more than %d ranked blocks", p->k, mcs::kMaxSelBlocks);
  if (c.empty) return ok();
  const size_t need = mcs::block_workspace_bytes(c.s);
  if (ws_bytes < need) return fail(MCS_ERR_WORKSPACE, "block workspace %zu < %zu bytes", ws_bytes, need);
  if (mcs_status s = check_ptrs({{Q, "Q", false}, {K, "K", false}, {perm, "perm", false}, {idx, "idx", false},
                                 {ws, "ws", false}}))
    return s;
  return hip_status(mcs::launch_block_select(c.s, c.bf16, Q, K, perm, idx, ws, (hipStream_t)stream),
                    "mcs_block_select");
}

mcs_status mcs_residual_drift(const mcs_problem* p, const void* Q, const void* K, const void* V, const void* O,
                              const int32_t* rows, int32_t n_rows, float* drift, void* ws, size_t ws_bytes,
                              void* stream) {
  Checked c;
  if (mcs_status s = check_problem(p, c)) return s;
  if (n_rows < 1 || n_rows > mcs::kMaxDriftRows)
    return fail(MCS_ERR_INVALID_ARG, "n_rows=%d outside [1, %d]", n_rows, mcs::kMaxDriftRows);
  if (c.empty) return ok();
  const size_t need = mcs::drift_workspace_bytes(c.s, n_rows);
  if (ws_bytes < need) return fail(MCS_ERR_WORKSPACE, "drift workspace %zu < %zu bytes", ws_bytes, need);
  if (mcs_status s = check_ptrs({{Q, "Q", false}, {K, "K", false}, {V, "V", false}, {O, "O", false},
                                 {rows, "rows", false}, {drift, "drift", false}, {ws, "ws", false}}))
    return s;
  return hip_status(mcs::launch_drift(c.s, c.bf16, Q, K, V, O, rows, n_rows, drift, ws, (hipStream_t)stream),
                    "mcs_residual_drift");
}

mcs_status mcs_residual_drift_noalloc(const mcs_problem* p, const void* Q, const void* K, const void* V,
                                      const void* O, const int32_t* rows, int32_t n_rows, float* drift,
                                      void* stream) {
  Checked c;
  if (mcs_status s = check_problem(p, c)) return s;
  if (n_rows < 1 || n_rows > mcs::kMaxDriftRows)
    return fail(MCS_ERR_INVALID_ARG, "n_rows=%d outside [1, %d]", n_rows, mcs::kMaxDriftRows);
  if (c.empty) return ok();
  const size_t need = mcs::drift_workspace_bytes(c.s, n_rows);
  if (need > kNoallocScratchBytes)
    return fail(MCS_ERR_WORKSPACE, "the check needs %zu bytes of scratch, more than the %zu of the static scratch",
                need, kNoallocScratchBytes);
  if (mcs_status s = check_ptrs({{Q, "Q", false}, {K, "K", false}, {V, "V", false}, {O, "O", false},
                                 {rows, "rows", false}, {drift, "drift", false}}))
    return s;
  void* ws = nullptr;
  if (mcs_status s = scratch_on_current_device(&ws)) return s;
  return hip_status(mcs::launch_drift(c.s, c.bf16, Q, K, V, O, rows, n_rows, drift, ws, (hipStream_t)stream),
                    "mcs_residual_drift_noalloc");
}

mcs_status mcs_sparse_attn(const mcs_problem* p, const void* Q, const void* K, const void* V,
                           const int32_t* perm, const int32_t* idx, const void* R, void* O,
                           void* stream) {
  Checked c;
  if (mcs_status s = check_problem(p, c)) return s;
  if (c.empty) return ok();
  if (mcs_status s = check_ptrs({{Q, "Q", false}, {K, "K", false}, {V, "V", false}, {perm, "perm", false},
                                 {idx, "idx", false}, {R, "R", true}, {O, "O", false}}))
    return s;
  if (O == Q || O == K || O == V || O == R)
    return fail(MCS_ERR_INVALID_ARG, "O aliases an input");
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = c.bf16 ? mcs::launch_sparse_bf16(c.s, Q, K, V, perm, idx, nullptr, (void*)R, c.r_f32, O, false, st)
                              : mcs::launch_sparse_f32(c.s, Q, K, V, perm, idx, (float*)R, O, false, st);
  return hip_status(e, "mcs_sparse_attn");
}

}  // extern "C"
