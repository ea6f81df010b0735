// Score-scan building blocks shared by the stand-alone score kernel and the
// fused decode pipeline (JSSA summary Figure 1 and section 3.1: every cached
// token is scored with the projected queries of its KV head's group against
// the projected-key cache).
//
// Layout of the scan: every lane issues U 16-byte loads of projected keys per
// workgroup step; a wave load covers TPW = 64/LPT whole tokens (LPT =
// R*bytes/16 lanes per token) and a step PER_ITER = 4 waves x U x TPW tokens.
//
// Two ways to form the scores, chosen by shape:
//  * matrix cores (bf16 or FP8 E4M3 keys, R = 32 or 64): 16 tokens' keys are
//    the B operand of v_mfma_f32_16x16x32_bf16 (bf16: lane l loads token
//    l % 16, elements 32 s + 8 (l / 16) .. +7 of K-step s); the A operand
//    holds the group's projected queries (row g = query head g; row 0 = the
//    group mean for the mean reduction), each fp32 coordinate split into three
//    bf16 terms whose sum is the coordinate, so the products see the full fp32
//    query.  FP8 keys are widened to bf16 in registers (exact) after 16-byte
//    loads of 16 codes: at R = 64 lane l loads elements 16 (l / 16) .. +15 of
//    token l % 16 (two K-steps of 8); at R = 32 a load covers 32 tokens (lane
//    l: token l % 16 + 16 (l / 32), elements 16 ((l / 16) % 2) .. +15) and a
//    v_permlane32_swap hands each half-wave the other half's second 8 codes,
//    so every lane holds 8 elements of one token for each of two 16-token
//    MFMAs; the query fragment follows the same element order;
//  * vector ALU (other shapes): each lane keeps its slice of the projected
//    queries in registers and the per-head dot products are completed with
//    DPP sums.
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
  static constexpr bool F8 = KPT == 2;                                      // FP8 E4M3 keys
  static constexpr bool MF = (KPT == 1 || KPT == 2) && (R == 32 || R == 64);  // matrix-core scoring
  static constexpr int KS = R / 32;                                          // K-steps per token (MF)
  static_assert(LPT >= 1 && LPT <= 16 && (LPT & (LPT - 1)) == 0, "lanes per token");
  static_assert(!MF || F8 || U % KS == 0, "a wave's loads cover whole 16-token groups");
  static_assert(!(MF && F8) || TPW == 16 || TPW == 32, "FP8 loads cover 16 or 32 tokens");
};

constexpr int kQTerms = 3;  // bf16 terms per fp32 query coordinate (matrix-core scoring)

// Token (offset within a workgroup step) and byte (within the token's row) of
// this lane's u-th load.
// (Waves 4 w' + j of a wider workgroup take the loads of wave j: the scores of
// a token do not depend on which wave forms them.)
template <int KPT, int R>
__device__ __forceinline__ int slot_token(int u) {
  using S = ScanShape<KPT, R>;
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3;
  if constexpr (S::MF && S::F8) return (wave * S::U + u) * S::TPW + (lane & 15) + (S::TPW == 32 ? 16 * (lane >> 5) : 0);
  else if constexpr (S::MF) return (wave * (S::U / S::KS) + u / S::KS) * 16 + (lane & 15);
  else return (wave * S::U + u) * S::TPW + lane / S::LPT;
}
template <int KPT, int R>
__device__ __forceinline__ int slot_byte(int u) {
  using S = ScanShape<KPT, R>;
  const int lane = threadIdx.x & 63;
  if constexpr (S::MF && S::F8) return 16 * ((lane >> 4) & (S::LPT - 1));
  else if constexpr (S::MF) return (32 * (u % S::KS) + 8 * (lane >> 4)) * 2;
  else return (lane % S::LPT) * 16;
}
// Contraction index of element j of lane group kg's 8-element slice in K-step s
// of the matrix-core scoring (the same for the key and the query operand).
template <int KPT, int R>
__device__ __forceinline__ int mf_index(int s, int kg, int j) {
  using S = ScanShape<KPT, R>;
  if constexpr (S::F8 && S::TPW == 16) return 16 * kg + 8 * s + j;              // R = 64
  else if constexpr (S::F8) return 16 * (kg & 1) + 8 * (kg >> 1) + j;           // R = 32
  else return 32 * s + 8 * kg + j;
}

// The group's projected queries as the scan uses them.
template <int KPT, int R, int GE, bool MF = ScanShape<KPT, R>::MF>
struct QFrag {
  float q[GE][ScanShape<KPT, R>::EPL];  // this lane's slice (vector ALU)
};
template <int KPT, int R, int GE>
struct QFrag<KPT, R, GE, true> {
  u32x4_t a[R / 32][kQTerms];  // A-operand fragments, one per K-step and term
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

// Projected queries (fp32, element g * R + i read through `ld`) into the
// scan's form.  Matrix cores: row m of the A operand is query head m (rows
// >= G are zero) or, for the mean (GE = 1), row 0 is the group mean formed as
// in load_qreg; each coordinate becomes kQTerms bf16 terms.
template <int KPT, int R, int GE, typename Ld>
__device__ __forceinline__ void load_qfrag(Ld ld, int G, QFrag<KPT, R, GE>& qf) {
  using S = ScanShape<KPT, R>;
  if constexpr (S::MF) {
    const int lane = threadIdx.x & 63, m = lane & 15, kg = lane >> 4;
    const float invG = 1.0f / float(G);
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = mf_index<KPT, R>(s, kg, j);
        x[j] = 0.f;
        if constexpr (GE == 1) {
          if (m == 0) {
            float sm = 0.f;
            for (int g = 0; g < G; ++g) sm += ld(g * R + i);
            x[j] = sm * invG;
          }
        } else {
          if (m < G) x[j] = ld(m * R + i);
        }
      }
      uint32_t w[4][kQTerms];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_bf16x2_terms<kQTerms>(x[2 * e], x[2 * e + 1], w[e]);
#pragma unroll
      for (int k = 0; k < kQTerms; ++k) qf.a[s][k] = u32x4_t{w[0][k], w[1][k], w[2][k], w[3][k]};
    }
  } else {
    load_qreg<KPT, R, GE>(ld, G, qf.q);
  }
}

// Scores of the tokens of one workgroup step from this lane's U loads
// (v[u] holds the 16 bytes at slot_token(u) / slot_byte(u)).  Calls
// emit(token offset within the step, score) once per token, in one lane.
// MAX over the G heads (GE = G) or the group-mean query (GE = 1).
//
// Matrix cores: a 16-token MFMA leaves the token scores in lanes 0..15 (row
// block 0 holds query heads 0..3; heads 4..7 come from lanes 16..31).  The
// scores of four such groups are moved into one register with lane swaps
// (v_permlane16_swap puts group 1 beside group 0, v_permlane32_swap the pair
// 2-3 beside 0-1), so each lane emits one token and the callers' per-token
// work runs once per 64 tokens with no divergent branch.
template <int KPT, int R, int GE, typename F>
__device__ __forceinline__ void score_loads(const uint4 (&v)[ScanShape<KPT, R>::U], const QFrag<KPT, R, GE>& qf,
                                            int G, F emit) {
  using S = ScanShape<KPT, R>;
  (void)G;  // GE == G for the max
  const int lane = threadIdx.x & 63;
  // group score in lanes 0..15: the max over the G heads' rows (or row 0)
  auto group_best = [&](const f32x4_t& c) {
    float best = c[0];
    if constexpr (GE > 1) {
#pragma unroll
      for (int i = 1; i < 4; ++i)
        if (i < GE) best = fmaxf(best, c[i]);
      if constexpr (GE > 4) best = xor16_max(best);
    }
    return best;
  };
  // lanes 16 q .. 16 q + 15 <- lanes 0..15 of b[q]
  auto gather4 = [](float b0, float b1, float b2, float b3) {
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(b0), __float_as_uint(b1), false, false);
    const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(b2), __float_as_uint(b3), false, false);
    const auto z = __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false);
    return __uint_as_float(z[0]);
  };
  if constexpr (S::MF) {
    const int wave = (threadIdx.x >> 6) & 3;
    if constexpr (S::F8 && S::TPW == 32) {
      // R = 32: one load = 32 tokens; the half-waves trade their second 8 codes
      static_assert(S::U % 2 == 0, "loads in pairs");
#pragma unroll
      for (int u = 0; u < S::U; u += 2) {
        float best[4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4& w = v[u + j];
          const auto x0 = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
          const auto x1 = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
          // tokens 0..15 and 16..31 of the load
          const u32x4_t b0 = e4m3x8_to_bf16(x0[0], x1[0]), b1 = e4m3x8_to_bf16(x0[1], x1[1]);
          f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < kQTerms; ++k) {
            c0 = mfma16(qf.a[0][k], b0, c0);
            c1 = mfma16(qf.a[0][k], b1, c1);
          }
          best[2 * j] = group_best(c0);
          best[2 * j + 1] = group_best(c1);
        }
        emit((wave * S::U + u) * 32 + lane, gather4(best[0], best[1], best[2], best[3]));
      }
    } else {
      // one 16-token group per F8 load (R = 64: two K-steps in it) or per KS
      // bf16 loads
      constexpr int NG = S::F8 ? S::U : S::U / S::KS;  // groups per step and wave
      static_assert(NG % 4 == 0 || NG == 2, "groups combine in fours or twos");
      float best[NG];
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
        if constexpr (S::F8) {
          const u32x4_t b[2] = {e4m3x8_to_bf16(v[q].x, v[q].y), e4m3x8_to_bf16(v[q].z, v[q].w)};
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int k = 0; k < kQTerms; ++k) c = mfma16(qf.a[s][k], b[s], c);
        } else {
#pragma unroll
          for (int s = 0; s < S::KS; ++s)
#pragma unroll
            for (int k = 0; k < kQTerms; ++k) c = mfma16(qf.a[s][k], as_u32x4(v[q * S::KS + s]), c);
        }
        best[q] = group_best(c);
      }
      if constexpr (NG % 4 == 0) {
#pragma unroll
        for (int q = 0; q < NG; q += 4)
          emit((wave * NG + q) * 16 + lane, gather4(best[q], best[q + 1], best[q + 2], best[q + 3]));
      } else {
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(best[0]), __float_as_uint(best[1]), false,
                                                        false);
        if (lane < 32) emit(wave * NG * 16 + lane, __uint_as_float(x[0]));
      }
    }
  } else {
    const int p = lane % S::LPT;
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const float best = score_of<KPT, R, GE>(v[u], qf.q);
      if (p == 0) emit(slot_token<KPT, R>(u), best);
    }
  }
}

}  // namespace jssa
