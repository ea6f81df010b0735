// Radix-select building blocks shared by the score kernel (first digit) and
// the selection kernels: histogram threshold search in shared memory.
#pragma once

#include "jssa_device.hpp"
#include "jssa_internal.hpp"

namespace jssa {

// In a shared-memory histogram of 256*BPT bins, find the bin that holds the
// need-th largest element (1 <= need <= total), counting from the highest bin
// down.  Writes the bin and the number of elements in higher bins to
// out[0], out[1] (shared memory).  All 256 threads must call it.
template <int BPT>
__device__ void find_bin_from_top(const uint32_t* hist, uint32_t need, uint32_t* scan_tmp,
                                  uint32_t* out) {
  static_assert(BPT >= 1 && (BPT & (BPT - 1)) == 0, "bins per thread: a power of two");
  const int seg = 255 - int(threadIdx.x);  // thread 0 owns the highest segment
  if (threadIdx.x == 0) { out[0] = 0u; out[1] = 0u; }  // defined result even if need > total
  uint32_t sum = 0;
  // bins summed from a per-thread rotation, so neighbouring lanes read different banks
#pragma unroll
  for (int j = 0; j < BPT; ++j) sum += hist[seg * BPT + ((j + int(threadIdx.x)) & (BPT - 1))];
  uint32_t total;
  const uint32_t above = block_exclusive_scan(sum, scan_tmp, &total);
  if (above < need && need <= above + sum) {
    uint32_t cum = above;
    for (int j = BPT - 1; j >= 0; --j) {
      const uint32_t c = hist[seg * BPT + j];
      if (cum + c >= need) {
        out[0] = uint32_t(seg * BPT + j);
        out[1] = cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

// Same, counting from the lowest bin up: the bin holding the need-th smallest
// element; out[1] = number of elements in lower bins.
template <int BPT>
__device__ void find_bin_from_bottom(const uint32_t* hist, uint32_t need, uint32_t* scan_tmp,
                                     uint32_t* out) {
  static_assert(BPT >= 1 && (BPT & (BPT - 1)) == 0, "bins per thread: a power of two");
  const int seg = int(threadIdx.x);
  if (threadIdx.x == 0) { out[0] = 0u; out[1] = 0u; }
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) sum += hist[seg * BPT + ((j + int(threadIdx.x)) & (BPT - 1))];
  uint32_t total;
  const uint32_t below = block_exclusive_scan(sum, scan_tmp, &total);
  if (below < need && need <= below + sum) {
    uint32_t cum = below;
    for (int j = 0; j < BPT; ++j) {
      const uint32_t c = hist[seg * BPT + j];
      if (cum + c >= need) {
        out[0] = uint32_t(seg * BPT + j);
        out[1] = cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

// Candidates of sequence b: t < max(T_b - W, 0), with T_b clamped to [0, t_max].
__device__ __forceinline__ int candidates_of(const int32_t* seq_lens, int b, int t_max, int window,
                                             int* Tb_out) {
  int Tb = seq_lens[b];
  Tb = Tb < 0 ? 0 : (Tb > t_max ? t_max : Tb);
  *Tb_out = Tb;
  const int n = Tb - window;
  return n > 0 ? n : 0;
}

constexpr int kKeysPerThread = kSelTile / 256;

// Keys of one selection tile, round-major: thread x holds tokens t0 + i*256 + x
// (coalesced loads, all issued before use).  Tokens past t_end repeat the last
// key and must be masked by the caller.
__device__ __forceinline__ void load_tile_keys(const float* srow, int t0, int t_end, uint32_t* key) {
  float v[kKeysPerThread];
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) v[i] = srow[min(t0 + i * 256 + int(threadIdx.x), t_end - 1)];
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) key[i] = score_key(v[i]);
}

// Last workgroup of a row after the first-digit histogram: moves the global
// histogram into `s_hist` (zeroing the global copy for the next call), finds
// the first-digit threshold bin of the k-th largest key and stores it in the
// row state.
__device__ __forceinline__ void finish_first_digit(uint32_t* g_hist, uint32_t* g_state,
                                                   uint32_t* s_hist, uint32_t* s_scan,
                                                   uint32_t* s_out, uint32_t need) {
  for (int i = threadIdx.x; i < kDigit1Bins; i += 256) {
    s_hist[i] = __hip_atomic_load(&g_hist[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&g_hist[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  find_bin_from_top<kDigit1Bins / 256>(s_hist, need, s_scan, s_out);
  if (threadIdx.x == 0) {
    g_state[RS_D1] = s_out[0];
    g_state[RS_NEED1] = need - s_out[1];
  }
}

}  // namespace jssa
