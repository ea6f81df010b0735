// Device-side helpers for the gfx950 kernels: element loads and conversions,
// cross-lane reductions with DPP, the order-preserving score key, and the
// release/acquire "last workgroup" ticket.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jssa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- elements ------------------------------------------------------------------
// DT = 0: float32, DT = 1: bfloat16 (stored as uint16 bit patterns).
template <int DT> struct Elem;
template <> struct Elem<0> { static constexpr int bytes = 4; static constexpr int per16 = 4; };
template <> struct Elem<1> { static constexpr int bytes = 2; static constexpr int per16 = 8; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Unpack one 16-byte vector into Elem<DT>::per16 floats (exact).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& v, float* out) {
  if constexpr (DT == 0) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  } else {
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x); out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z); out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  }
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Scalar element load with a run-time dtype (prologues only).
__device__ __forceinline__ float load_elem(const void* base, size_t i, int dt) {
  if (dt == 0) return reinterpret_cast<const float*>(base)[i];
  return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(base)[i]) << 16);
}

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ---- cross-lane reductions --------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
// DPP controls (gfx9): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppXor1 = 0xb1;
constexpr int kDppXor2 = 0x4e;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Sum over aligned groups of N lanes (N a power of two <= 64); every lane of
// the group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// ---- order-preserving key of an fp32 score ------------------------------------------
// Larger score <=> larger key.  -0.0 and +0.0 map to the same key; every NaN maps
// to 0, below -inf (0x007fffff), so NaNs rank last and tie among themselves.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- last-workgroup ticket ----------------------------------------------------------
// Every thread of the workgroup calls this after its global writes.  Returns
// true in exactly one workgroup of the `expected` that share `counter`: the
// last to arrive, which then sees every other workgroup's writes.  The counter
// is reset to zero for the next call.
__device__ __forceinline__ bool last_arrival(uint32_t* counter, uint32_t expected) {
  __shared__ uint32_t s_ticket;
  __threadfence();  // release this thread's writes at device scope
  __syncthreads();
  if (threadIdx.x == 0) s_ticket = atomicAdd(counter, 1u);
  __syncthreads();
  const bool last = (s_ticket == expected - 1);
  if (last) {
    __threadfence();  // acquire the other workgroups' writes
    if (threadIdx.x == 0) atomicExch(counter, 0u);
  }
  return last;
}

// Block-wide exclusive prefix sum of one value per thread (blockDim.x == 256).
// `tmp` is 256 words of shared memory; returns the exclusive prefix, and the
// total through `total`.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    uint32_t add = (t >= off) ? tmp[t - off] : 0u;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  uint32_t incl = tmp[t];
  *total = tmp[255];
  __syncthreads();
  return incl - v;
}

}  // namespace jssa
