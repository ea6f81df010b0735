// Head-shared soft voting (JSSA summary section E.3 compares it with the
// method's per-KV-head sets): every KV head votes with the softmax of its
// scaled scores over the sequence's candidates, the votes are summed over the
// KV heads, and one top-k of the vote is shared by all of them.
//
//  vote_partial_kernel: per (sequence, KV head, chunk of kVoteChunk
//    candidates) the running max m and sum l of exp2(x - m), x = s * scale *
//    log2(e) (NaN scores are skipped);
//  vote_kernel: per sequence and 1024-token tile, each KV head's partials
//    merged (one wave per head) into (M_h, L_h), then
//    vote[t] = sum_h exp2(x_ht - M_h) / L_h over the tile's candidates, and
//    the sequence's vote range;
//  vote_spread_kernel: an increasing map of the votes onto the exponent
//    range, for the selection's radix digits;
//  share_kernel: the sequence's index list copied to every KV head.
#include "jssa_device.hpp"
#include "jssa_internal.hpp"
#include "select_common.hpp"

namespace jssa {

struct VoteArgs {
  const float* scores;     // [B][Hkv][t_max]
  const int32_t* seq_lens;
  float* part;             // [B][Hkv][n_chunks][2]
  float* vote;             // [B][t_max]
  uint32_t* range;         // [B][2]: ~bits of the smallest vote, bits of the largest (zero on entry and exit)
  int Hkv, t_max, window, n_chunks;
  float l2scale;           // scale * log2(e)
};

// (m, l) of two parts: l sums exp2(x - m) over each part
__device__ __forceinline__ void ml_merge(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  l = (m == -INFINITY ? 0.f : l * exp2f(m - M)) + (m2 == -INFINITY ? 0.f : l2 * exp2f(m2 - M));
  m = M;
}

__global__ __launch_bounds__(256) void vote_partial_kernel(VoteArgs a) {
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  const int t0 = chunk * kVoteChunk, t1 = min(t0 + kVoteChunk, n_cand);
  const float* srow = a.scores + (size_t(b) * a.Hkv + h) * a.t_max;
  float m = -INFINITY, l = 0.f;
  for (int t = t0 + int(threadIdx.x); t < t1; t += 256) {
    const float x = a.l2scale * srow[t];
    if (x != x) continue;  // NaN: no vote
    if (x > m) {
      l = (m == -INFINITY ? 0.f : l * exp2f(m - x)) + 1.f;
      m = x;
    } else {
      l += exp2f(x - m);
    }
  }
  __shared__ float s_m[4], s_l[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    ml_merge(m, l, m2, l2);
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = l;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = s_m[0], L = s_l[0];
    for (int w = 1; w < 4; ++w) ml_merge(M, L, s_m[w], s_l[w]);
    float* p = a.part + ((size_t(b) * a.Hkv + h) * a.n_chunks + chunk) * 2;
    p[0] = M;
    p[1] = L;
  }
}

__global__ __launch_bounds__(256) void vote_kernel(VoteArgs a) {
  const int tile = blockIdx.x, b = blockIdx.y;
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  const int t0 = tile * 1024;
  if (t0 >= n_cand) return;
  __shared__ float s_M[kVoteMaxHeads], s_L[kVoteMaxHeads];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_chunks_b = (n_cand + kVoteChunk - 1) / kVoteChunk;
  for (int h = wave; h < a.Hkv; h += 4) {
    const float* p = a.part + (size_t(b) * a.Hkv + h) * a.n_chunks * 2;
    float m = -INFINITY, l = 0.f;
    for (int c = lane; c < n_chunks_b; c += 64) ml_merge(m, l, p[2 * c], p[2 * c + 1]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
      ml_merge(m, l, m2, l2);
    }
    if (lane == 0) {
      s_M[h] = m;
      s_L[h] = l;
    }
  }
  __syncthreads();
  const int t1 = min(t0 + 1024, n_cand);
  uint32_t lo = 0xffffffffu, hi = 0u;  // vote bits (votes are >= 0, so bits order as values)
  for (int t = t0 + int(threadIdx.x); t < t1; t += 256) {
    float v = 0.f;
    for (int h = 0; h < a.Hkv; ++h) {
      const float x = a.l2scale * a.scores[(size_t(b) * a.Hkv + h) * a.t_max + t];
      v += (x != x || s_L[h] == 0.f) ? 0.f : exp2f(x - s_M[h]) / s_L[h];
    }
    a.vote[size_t(b) * a.t_max + t] = v;
    lo = min(lo, v > 0.f ? __float_as_uint(v) : 0xffffffffu);  // the smallest positive vote
    hi = max(hi, __float_as_uint(v));
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    atomicMax(&a.range[2 * b], ~lo);  // the complement: zero (the state between calls) is "none yet"
    atomicMax(&a.range[2 * b + 1], hi);
  }
}

// The votes of a sequence lie within a narrow range (each head's votes sum
// to one over ~T_b tokens), so their float keys would share a few top-digit
// bins of the selection's histogram.  Each positive vote is replaced by
//   exp2(250 u - 125),  u = log2(v / v_min) / log2(v_max / v_min)
// (v_min the smallest positive vote; zero stays zero): increasing in v up to
// fp32 rounding, it spreads the sequence's range, outliers included, over the
// normal exponent range.
__global__ __launch_bounds__(256) void vote_spread_kernel(VoteArgs a) {
  const int tile = blockIdx.x, b = blockIdx.y;
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  const int t0 = tile * 1024;
  if (t0 >= n_cand) return;
  const uint32_t lo = ~a.range[2 * b];
  const float vmax = __uint_as_float(a.range[2 * b + 1]);
  const float l_min = lo == 0xffffffffu ? 0.f : __log2f(__uint_as_float(lo));
  const float span = lo == 0xffffffffu ? 0.f : __log2f(vmax) - l_min;
  const float k = span > 0.f ? 250.f / span : 0.f;
  const int t1 = min(t0 + 1024, n_cand);
  for (int t = t0 + int(threadIdx.x); t < t1; t += 256) {
    float* p = a.vote + size_t(b) * a.t_max + t;
    const float v = *p;
    *p = v > 0.f ? exp2f(k * (__log2f(v) - l_min) - 125.f) : 0.f;
  }
}

// idx[b, h, i] = shared[b, i] for i < n, n_sel[b, h] = n (n = shared_n[b]);
// the sequence's vote range is reset for the next call
__global__ __launch_bounds__(256) void share_kernel(const int32_t* shared, const int32_t* shared_n, int32_t* idx,
                                                    int32_t* n_sel, uint32_t* range, int Hkv, int S) {
  const int h = blockIdx.y, b = blockIdx.z;
  int n = shared_n[b];
  n = n < 0 ? 0 : (n > S ? S : n);
  const int i = blockIdx.x * 256 + int(threadIdx.x);
  if (i < n) idx[(size_t(b) * Hkv + h) * S + i] = shared[size_t(b) * S + i];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    n_sel[size_t(b) * Hkv + h] = n;
    if (h == 0) {
      range[2 * b] = 0u;
      range[2 * b + 1] = 0u;
    }
  }
}

jssa_desc vote_desc(const jssa_desc& d) {
  jssa_desc v = d;
  v.n_q_heads = 1;
  v.n_kv_heads = 1;
  v.reduce = JSSA_REDUCE_MAX;
  return v;
}

hipError_t launch_vote_select(const jssa_desc& d, const float* scores, const int32_t* seq_lens, int32_t* idx,
                              int32_t* n_sel, char* ws_base, const Workspace& ws, hipStream_t s) {
  VoteArgs a;
  a.scores = scores; a.seq_lens = seq_lens;
  a.part = reinterpret_cast<float*>(ws_base + ws.vote_part);
  a.vote = reinterpret_cast<float*>(ws_base + ws.vote);
  a.range = reinterpret_cast<uint32_t*>(ws_base + ws.vote_range);
  a.Hkv = d.n_kv_heads; a.t_max = d.t_max; a.window = d.window;
  a.n_chunks = (d.t_max + kVoteChunk - 1) / kVoteChunk;
  a.l2scale = d.scale * kLog2e;
  hipLaunchKernelGGL(vote_partial_kernel, dim3(a.n_chunks, d.n_kv_heads, d.batch), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vote_kernel, dim3((d.t_max + 1023) / 1024, d.batch), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vote_spread_kernel, dim3((d.t_max + 1023) / 1024, d.batch), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the shared selection: the stand-alone top-k of the vote (one "KV head")
  const jssa_desc vd = vote_desc(d);
  Workspace nested;
  if (!workspace_layout(vd, JSSA_OP_TOPK, &nested)) return hipErrorInvalidValue;
  // the nested top-k workspace, addressed from this one's base, with this one's
  // queue (its diagnostics are reported with the vote's)
  const Workspace lt = rebase_workspace(nested, ws.vote_topk, ws.queue);
  char* tbase = ws_base;
  int32_t* sidx = reinterpret_cast<int32_t*>(ws_base + ws.vote_idx);
  int32_t* sn = reinterpret_cast<int32_t*>(ws_base + ws.vote_nsel);
  e = launch_hist(vd, a.vote, seq_lens, tbase, lt, s);
  if (e == hipSuccess) e = launch_candidates(vd, a.vote, seq_lens, tbase, lt, s);
  if (e == hipSuccess)
    e = launch_resolve_attend(vd, true, false, nullptr, nullptr, nullptr, sidx, sn, seq_lens, nullptr, nullptr,
                              tbase, lt, s);
  if (e != hipSuccess) return e;
  const int S = d.topk + d.window;
  hipLaunchKernelGGL(share_kernel, dim3((S + 255) / 256, d.n_kv_heads, d.batch), dim3(256), 0, s, sidx, sn, idx,
                     n_sel, a.range, d.n_kv_heads, S);
  return hipGetLastError();
}

}  // namespace jssa
