// Device-side helpers shared by the gfx950 kernels: vector types, MFMA
// wrappers, cross-lane exchange, LDS transpose reads, XCD-aware block mapping.
//
// Register layouts used throughout (checked on gfx950 hardware):
//  v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//    A: lane l holds row l%32, k = 8*(l/32) + j  (j = 0..7)
//    B: lane l holds col l%32, k = 8*(l/32) + j
//    D: lane l element i is row 8*(i/4) + 4*(l/32) + i%4, col l%32
//  ds_read_b64_tr_b16: in each group of 16 lanes, lane i element j receives
//    element i%4 of the 8-byte row addressed by lane 4*j + i/4 of the group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kInf = __builtin_huge_valf();

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane l^32 (exchange of the two wave halves).
__device__ __forceinline__ float partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((lane_id() & 32) ? r[0] : r[1]);
}

// max / sum of a lane's value and its partner's (lane l^32).  The swap
// returns the low-half value in r[0] and the high-half value in r[1] on every
// lane, so no select is needed, and both halves get the same bits.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposing 8-byte LDS read (see the layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr(const void* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Keys [0, limit) are visible to the query at position q_offset + qpos:
// everything without a causal block, else every key up to the end of the
// query's frame block (clamped to Nkv).  Nondecreasing in qpos.
__device__ __forceinline__ int visible_limit(int qpos, int causal_block, int q_offset, int Nkv) {
  if (!causal_block) return Nkv;
  const long long lim = ((long long)(q_offset + qpos) / causal_block + 1) * causal_block;
  return lim < Nkv ? (int)lim : Nkv;
}

// Workgroups are dealt round-robin to the 8 XCDs in launch order.  Give each
// XCD a contiguous range of logical work units so that units sharing K/V
// (neighbouring query tiles or groups of one head) share that XCD's L2.
// The grid must be launched with 8 * per_xcd blocks; ids beyond the real
// unit count are returned as-is and must be skipped by the caller.
__device__ __forceinline__ int xcd_unit(int bid, int per_xcd) { return (bid & 7) * per_xcd + (bid >> 3); }

// Monotone map of a float to an unsigned key (total order, -0 == +0 assumed
// normalised by the caller).
__device__ __forceinline__ uint32_t float_order_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over one 64-lane wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (l >= o) v += t;
  }
  return v;
}

// fp64 value of another lane by a DPP pattern (both 32-bit halves moved).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

__device__ __forceinline__ double partner32_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  auto lo = __builtin_amdgcn_permlane32_swap((unsigned)u, (unsigned)u, false, false);
  auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
  const bool up = lane_id() & 32;
  const unsigned l = up ? lo[0] : lo[1], h = up ? hi[0] : hi[1];
  return __longlong_as_double((long long)(((unsigned long long)h << 32) | l));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// fp32 sum over the 64 lanes, returned in every lane (same pattern as below).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  v += __shfl_xor(v, 16, 64);
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the 64 lanes, returned in every lane: DPP within rows of 16
// (quad swaps, half-row and row mirrors), then the row pairs and the halves.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  v += __shfl_xor(v, 16, 64);
  v += partner32_f64(v);
  return v;
}

// Raise a kernel's dynamic-LDS limit (host side; done once per kernel).
inline bool allow_dynamic_lds(const void* kernel, int bytes) {
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  (void)hipGetLastError();
  return e == hipSuccess;
}

}  // namespace mcs
