// Score-scan building blocks shared by the stand-alone score kernel and the
// fused decode pipeline (JSSA summary Figure 1 and section 3.1: every cached
// token is scored with the projected queries of its KV head's group against
// the projected-key cache).
//
// Layout of the scan: a token's projected key (R elements) is spread over
// LPT = R*bytes/16 lanes (one 16-byte load each); each lane keeps the matching
// slice of the group's projected queries in registers and the per-head dot
// products are completed with DPP sums.  A wave covers TPW = 64/LPT tokens
// per load, a workgroup step covers PER_ITER = 4 waves x U loads.
#pragma once

#include "jssa_device.hpp"
#include "jssa_internal.hpp"

namespace jssa {

template <int KPT, int R>
struct ScanShape {
  static constexpr int EB = Elem<KPT>::bytes;
  static constexpr int EPL = Elem<KPT>::per16;
  static constexpr int LPT = R / EPL;
  static constexpr int TPW = 64 / LPT;
  static constexpr int U = JSSA_SCORE_UNROLL;
  static constexpr int PER_ITER = 4 * TPW * U;
  static_assert(LPT >= 1 && LPT <= 16 && (LPT & (LPT - 1)) == 0, "lanes per token");
};

// Projected queries of KV head h's group, fp32, into s_qp[g * R + i]:
//   qp[g][i] = sum_d q[b, h*G + g, d] * P[h, d, i]
// The query rows are staged in shared memory; the d-sum of each output is
// split over several threads when G*R < 256 and the parts are added in a
// fixed order.  s_q: G*d_k floats, s_part: 512 floats, s_qp: G*R floats.
template <int R>
__device__ void project_group_query(const void* q, int q_dtype, const float* P, int Hq, int d_k,
                                    int G, int b, int h, float* s_q, float* s_part, float* s_qp) {
  const size_t q0 = (size_t(b) * Hq + size_t(h) * G) * d_k;
  for (int i = threadIdx.x; i < G * d_k; i += 256) s_q[i] = load_elem(q, q0 + i, q_dtype);
  __syncthreads();
  const int GR = G * R;
  const int parts = GR >= 256 ? 1 : 256 / GR;
  const int dper = d_k / parts;
  const float* Ph = P + size_t(h) * d_k * R;
  for (int j = threadIdx.x; j < GR * parts; j += 256) {
    const int o = j % GR, part = j / GR;
    const int g = o / R, i = o - g * R;
    const float* qg = s_q + g * d_k;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int d = part * dper; d < (part + 1) * dper; d += 4) {
      a0 = fmaf(qg[d + 0], Ph[size_t(d + 0) * R + i], a0);
      a1 = fmaf(qg[d + 1], Ph[size_t(d + 1) * R + i], a1);
      a2 = fmaf(qg[d + 2], Ph[size_t(d + 2) * R + i], a2);
      a3 = fmaf(qg[d + 3], Ph[size_t(d + 3) * R + i], a3);
    }
    s_part[j] = (a0 + a1) + (a2 + a3);
  }
  __syncthreads();
  for (int o = threadIdx.x; o < GR; o += 256) {
    float acc = 0.f;
    for (int part = 0; part < parts; ++part) acc += s_part[part * GR + o];
    s_qp[o] = acc;
  }
  __syncthreads();
}

// This lane's slice of the projected queries: qreg[g][e] = qp[g][p*EPL + e]
// (GE = G for the group max), or of their mean (GE = 1).  qp may be shared or
// global memory; `ld` reads one float.
template <int KPT, int R, int GE, typename Ld>
__device__ __forceinline__ void load_qreg(Ld ld, int G, float (&qreg)[GE][ScanShape<KPT, R>::EPL]) {
  using S = ScanShape<KPT, R>;
  const int p = (threadIdx.x & 63) % S::LPT;
  if constexpr (GE == 1) {
    const float invG = 1.0f / float(G);
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) {
      float sm = 0.f;
      for (int g = 0; g < G; ++g) sm += ld(g * R + p * S::EPL + e);
      qreg[0][e] = sm * invG;
    }
  } else {
#pragma unroll
    for (int g = 0; g < GE; ++g)
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) qreg[g][e] = ld(g * R + p * S::EPL + e);
  }
}

// Score of the token whose 16-byte slice this lane holds (valid in every lane
// of the token's LPT-lane group after the DPP sums).
template <int KPT, int R, int GE>
__device__ __forceinline__ float score_of(const uint4& raw, const float (&qreg)[GE][ScanShape<KPT, R>::EPL]) {
  using S = ScanShape<KPT, R>;
  float kv[S::EPL];
  unpack16<KPT>(raw, kv);
  float best;
#pragma unroll
  for (int g = 0; g < GE; ++g) {
    float dsum = 0.f;
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) dsum = fmaf(qreg[g][e], kv[e], dsum);
    dsum = group_sum<S::LPT>(dsum);
    best = (g == 0) ? dsum : fmaxf(best, dsum);
  }
  return best;
}

// Scores NIT workgroup steps of logical tokens [i0, i0 + NIT*PER_ITER): logical
// token i is cached token tok(i) (clamped to a valid token by the caller) and
// is real when i < i_end.  key[it][u] receives the order-preserving key of
// logical token i0 + it*PER_ITER + (wave*U + u)*TPW + tw in every lane of its
// group.  Loads are double-buffered across steps and issued without per-lane
// branches.
template <int KPT, int R, int GE, int NIT, typename Tok>
__device__ __forceinline__ void score_steps(const char* kp_row, Tok tok, int i0, int i_end,
                                            const float (&qreg)[GE][ScanShape<KPT, R>::EPL],
                                            uint32_t (&key)[NIT][ScanShape<KPT, R>::U]) {
  using S = ScanShape<KPT, R>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane % S::LPT, tw = lane / S::LPT;
  auto load_step = [&](int it, uint4* v) {
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int i = min(i0 + it * S::PER_ITER + (wave * S::U + u) * S::TPW + tw, i_end - 1);
      v[u] = load16_nt(kp_row + (size_t(tok(i)) * R + p * S::EPL) * S::EB);
    }
  };
  uint4 cur[S::U];
  load_step(0, cur);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    uint4 nxt[S::U];
    if (it + 1 < NIT) load_step(it + 1, nxt);
#pragma unroll
    for (int u = 0; u < S::U; ++u) key[it][u] = score_key(score_of<KPT, R, GE>(cur[u], qreg));
    if (it + 1 < NIT) {
#pragma unroll
      for (int u = 0; u < S::U; ++u) cur[u] = nxt[u];
    }
  }
}

// Same keys as score_steps, but every load of the NIT steps is issued before
// the first one is used: for scattered, latency-bound reads (a strided sample
// of a row) where one round trip per NIT steps beats one per step.
template <int KPT, int R, int GE, int NIT, typename Tok>
__device__ __forceinline__ void score_block(const char* kp_row, Tok tok, int i0, int i_end,
                                            const float (&qreg)[GE][ScanShape<KPT, R>::EPL],
                                            uint32_t (&key)[NIT][ScanShape<KPT, R>::U]) {
  using S = ScanShape<KPT, R>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane % S::LPT, tw = lane / S::LPT;
  uint4 v[NIT][S::U];
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int i = min(i0 + it * S::PER_ITER + (wave * S::U + u) * S::TPW + tw, i_end - 1);
      v[it][u] = load16_nt(kp_row + (size_t(tok(i)) * R + p * S::EPL) * S::EB);
    }
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int u = 0; u < S::U; ++u) key[it][u] = score_key(score_of<KPT, R, GE>(v[it][u], qreg));
}

}  // namespace jssa
