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
// DT = 0: float32, DT = 1: bfloat16 (stored as uint16 bit patterns), DT = 2:
// FP8 E4M3 (OCP E4M3: bias 7, largest value 448, no infinity; the projected
// scoring cache only).
template <int DT> struct Elem;
template <> struct Elem<0> { static constexpr int bytes = 4; static constexpr int per16 = 4; };
template <> struct Elem<1> { static constexpr int bytes = 2; static constexpr int per16 = 8; };
template <> struct Elem<2> { static constexpr int bytes = 1; static constexpr int per16 = 16; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// Two E4M3 codes (byte 2*HI and 2*HI+1 of w) -> their values; every E4M3
// value is a float (gfx950 reads the OCP encoding).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ f32x2_t e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}
// Four E4M3 codes (a word) -> four bfloat16 values in two words (exact: an
// E4M3 value has 4 significant bits and an exponent inside bfloat16's range).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
struct u32pair {
  uint32_t lo, hi;  // codes 0-1 and 2-3
};
__device__ __forceinline__ u32pair e4m3x4_to_bf16(uint32_t w) {
  return {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}
// Eight E4M3 codes (two words) -> the 8-element bf16 operand of one K-step.
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const u32pair a = e4m3x4_to_bf16(w0), b = e4m3x4_to_bf16(w1);
  return u32x4_t{a.lo, a.hi, b.lo, b.hi};
}
// float -> E4M3 code, round to nearest, ties to even, saturating at +-448 (the
// conversion instruction rounds to nearest even; the clamp makes magnitudes
// past 448 saturate instead of becoming NaN).  NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float f) {
  const float c = (f != f) ? f : fminf(fmaxf(f, -448.f), 448.f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0u, false) & 0xffu;
}

// Unpack one 16-byte vector into Elem<DT>::per16 floats (exact).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& v, float* out) {
  if constexpr (DT == 0) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  } else if constexpr (DT == 2) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t a = e4m3x2_to_f32<false>(w[i]), b = e4m3x2_to_f32<true>(w[i]);
      out[4 * i + 0] = a.x; out[4 * i + 1] = a.y; out[4 * i + 2] = b.x; out[4 * i + 3] = b.y;
    }
  } else {
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x); out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z); out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  }
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// 16-byte load with the nontemporal hint: for data streamed once (the
// projected-key scan, K/V rows), so it does not displace reusable lines.
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- matrix cores ------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies row m = l % 16 of A and
// column n = l % 16 of B, each with the eight contraction indices
// 8 (l / 16) .. 8 (l / 16) + 7 (element j of the 16-byte operand = index
// 8 (l / 16) + j); it receives column n = l % 16, rows 4 (l / 16) .. +3 of
// the 16 x 16 fp32 result.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ u32x4_t as_u32x4(const uint4& v) { return u32x4_t{v.x, v.y, v.z, v.w}; }

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

// Two floats -> packed bfloat16 (x0 in bits 0..15), round to nearest even, in
// one instruction (v_cvt_pk_bf16_f32).  For operands of the matrix cores.
__device__ __forceinline__ uint32_t pack_bf16x2(float x0, float x1) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t h = {(__bf16)x0, (__bf16)x1};
  return __builtin_bit_cast(uint32_t, h);
}

// (x0, x1) as sums of N packed bfloat16 terms, each the nearest bf16 to what
// the earlier terms leave (every remainder is exact in fp32).  N = 2 keeps
// about 16 significant bits, N = 3 all 24.
template <int N>
__device__ __forceinline__ void split_bf16x2_terms(float x0, float x1, uint32_t (&w)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    w[i] = pack_bf16x2(x0, x1);
    x0 -= __uint_as_float(w[i] << 16);
    x1 -= __uint_as_float(w[i] & 0xffff0000u);
  }
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

// Lanes l and l ^ 16 (l ^ 32) combined through the lane swaps of gfx950:
// with both operands equal, v_permlane16_swap returns the lower and the upper
// row of each 32-lane half (v_permlane32_swap: the lower and the upper half),
// so their sum (max) is the pair's sum (max) in both lanes -- a VALU op, no
// trip through the shared-memory crossbar.  The same value as v + shfl_xor(v,
// 16) in either lane (addition and fmaxf are commutative).
__device__ __forceinline__ float xor16_add(float v) {
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float xor32_add(float v) {
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Sum over aligned groups of N lanes (N a power of two <= 64); every lane of
// the group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  if constexpr (N >= 32) v = xor16_add(v);
  if constexpr (N >= 64) v = xor32_add(v);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  if constexpr (N >= 32) v = xor16_max(v);
  if constexpr (N >= 64) v = xor32_max(v);
  return v;
}

// Sum over lanes l ^ m for m = F, 2F, ..., 32 (F a power of two): the
// lane groups of F lanes that hold the same positions of different rows.
template <int F>
__device__ __forceinline__ float sum_across_groups(float v) {
#pragma unroll
  for (int off = F; off < 16; off <<= 1) v += __shfl_xor(v, off);
  if constexpr (F <= 16) v = xor16_add(v);
  if constexpr (F <= 32) v = xor32_add(v);
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

// ---- cross-workgroup hand-off -------------------------------------------------------
// Data one workgroup leaves for the last workgroup of its row is written with
// device-scope atomic stores (`publish`, which write through to the level that
// is coherent across XCDs) and read back with device-scope atomic loads
// (`consume`).  That avoids a device-scope release fence, which on gfx950 would
// write back the whole L2 of the XCD once per workgroup.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float consume(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t consume(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t consume(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread of the workgroup calls this after its publish() stores and
// device atomics.  It waits until they have completed, then takes a ticket;
// returns true in exactly one of the `expected` workgroups sharing `counter`:
// the last to arrive, which can then consume() everything the others
// published.  The counter is reset to zero for the next call.
__device__ __forceinline__ bool last_arrival(uint32_t* counter, uint32_t expected) {
  __shared__ uint32_t s_ticket;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's memory operations have completed
  __syncthreads();
  if (threadIdx.x == 0)
    s_ticket = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const bool last = (s_ticket == expected - 1);
  if (last && threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// ---- wave-wide scans and reductions through DPP ---------------------------------------
// Row shifts by 1, 2, 4 and 8 give the inclusive scan inside each row of 16
// lanes; the last lane of rows 0 and 2 is then broadcast into rows 1 and 3
// (row_bcast:15), and lane 31 into rows 2 and 3 (row_bcast:31).  Lanes whose
// source is outside the row take the operation's identity.
template <typename Op>
__device__ __forceinline__ uint32_t dpp_scan(uint32_t x, uint32_t id, Op op) {
  x = op(x, uint32_t(__builtin_amdgcn_update_dpp(int(id), int(x), 0x111, 0xf, 0xf, false)));
  x = op(x, uint32_t(__builtin_amdgcn_update_dpp(int(id), int(x), 0x112, 0xf, 0xf, false)));
  x = op(x, uint32_t(__builtin_amdgcn_update_dpp(int(id), int(x), 0x114, 0xf, 0xf, false)));
  x = op(x, uint32_t(__builtin_amdgcn_update_dpp(int(id), int(x), 0x118, 0xf, 0xf, false)));
  x = op(x, uint32_t(__builtin_amdgcn_update_dpp(int(id), int(x), 0x142, 0xa, 0xf, false)));
  x = op(x, uint32_t(__builtin_amdgcn_update_dpp(int(id), int(x), 0x143, 0xc, 0xf, false)));
  return x;
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  return dpp_scan(x, 0u, [](uint32_t u, uint32_t v) { return u + v; });
}
// Minimum / maximum over the 64 lanes (the same value in every lane).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = dpp_scan(x, 0xffffffffu, [](uint32_t u, uint32_t v) { return u < v ? u : v; });
  return uint32_t(__builtin_amdgcn_readlane(int(x), 63));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = dpp_scan(x, 0u, [](uint32_t u, uint32_t v) { return u > v ? u : v; });
  return uint32_t(__builtin_amdgcn_readlane(int(x), 63));
}

// Block-wide exclusive prefix sum of one value per thread (blockDim.x == 64 NW):
// a DPP scan inside each wave, then the NW wave totals through `tmp`
// (at least NW words of shared memory).  Returns the exclusive prefix and the
// block total through `total`.
template <int NW = 4>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_scan_incl(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = tmp[w];
    before += (w < wave) ? c : 0u;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

}  // namespace jssa
