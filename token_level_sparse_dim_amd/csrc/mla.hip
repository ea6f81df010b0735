// MLA layout (JSSA summary section 3.3): every token has one shared latent
// row of 576 elements (512 latent + 64 rotary) that serves as the key of all
// query heads, and whose first 512 elements are the value; selection yields
// one index set per sequence.  With G = Hq query heads per row, both
// contractions are matrix products and run on the gfx950 matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//
//  * scoring (JSSA summary Figure 1, sections 3.1 and 3.2): the per-head
//    scores of a token are the [Hq x r] projected queries times the token's
//    projected key; the MAX reduction takes the largest over the heads.  The
//    projected queries are fp32; each is split into two bf16 terms
//    (hi = rne(x), lo = rne(x - hi)) and both terms are multiplied with the
//    bf16 projected keys, so a score carries about 16 significant bits of each
//    query coordinate (|error| <= 2^-17 * sum_i |qp_i Kp_i|).
//  * attention over the selected rows: S^T = K_sel Q^T, an online softmax per
//    head, and O += P V_sel, with P split into bf16 hi + lo terms in the same
//    way (V is exact in bf16).
//
// (Operand layout of v_mfma_f32_16x16x32_bf16: see mfma16 in jssa_device.hpp.)
#include <hip/hip_ext.h>

#include "append_core.hpp"
#include "jssa_device.hpp"
#include "jssa_internal.hpp"
#include "select_common.hpp"

namespace jssa {

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ float mla_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> (hi, lo) bf16 pair with hi = rne(x), lo = rne(x - hi); x - hi is exact.
__device__ __forceinline__ void split_bf16(float x, uint16_t* hi, uint16_t* lo) {
  uint32_t w[2];
  split_bf16x2_terms<2>(x, 0.f, w);
  *hi = uint16_t(w[0]);
  *lo = uint16_t(w[1]);
}

// =====================================================================================
// Query projection: qp = q P (fp32), stored as bf16 hi / lo A-operand fragments.
// Fragment (b, mt, s, split) holds rows 16 mt .. 16 mt + 15 (query heads) and
// contraction indices 32 s .. 32 s + 31 (projection coordinates), 16 bytes per
// lane in lane order, so one wave loads it with one coalesced 16-byte load.
// =====================================================================================
struct MlaQArgs {
  const uint16_t* q;  // [B][Hq][576]
  const float* P;     // [576][R]
  uint16_t* qf;       // fragments [B][MT][R/32][2][64 lanes][8]
  int Hq, MT;
};

template <int R>
__device__ __forceinline__ size_t qfrag_at(int b, int MT, int mt, int m, int r, int split) {
  constexpr int KS = R / 32;
  const int s = r >> 5, kk = r & 31;
  const int lane = m + 16 * (kk >> 3);
  return ((((size_t(b) * MT + mt) * KS + s) * 2 + split) * 64 + lane) * 8 + (kk & 7);
}

// MAX: one wave per (16 query heads, 16 projection coordinates), on the
// matrix cores: A = the bf16 query rows (exact), B = P[:, 16 coordinates]
// split into bf16 hi + lo terms, so qp = q P_hi + q P_lo with fp32
// accumulation (|P - P_hi - P_lo| <= 2^-17 |P|).  All loads are issued
// before the first product.
template <int R>
__device__ __forceinline__ void qproj_wave(const MlaQArgs& a, int mt, int nt, int b, int lane) {
  constexpr int KS = kMlaDk / 32;
  const int g = lane >> 4, n16 = lane & 15;
  const uint16_t* qrow = a.q + (size_t(b) * a.Hq + 16 * mt + n16) * kMlaDk + 8 * g;
  const float* pcol = a.P + 16 * nt + n16;
  u32x4_t qa[KS];
  float pv[KS][8];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qa[s] = ld16(qrow + 32 * s);
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[s][j] = pcol[size_t(32 * s + 8 * g + j) * R];
  }
  f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint32_t w[4][2];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_bf16x2_terms<2>(pv[s][2 * e], pv[s][2 * e + 1], w[e]);
#pragma unroll
    for (int k = 0; k < 2; ++k) c = mfma16(qa[s], u32x4_t{w[0][k], w[1][k], w[2][k], w[3][k]}, c);
  }
  // result lane: coordinate 16 nt + n16, query heads 16 mt + 4 g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint16_t hi, lo;
    split_bf16(c[i], &hi, &lo);
    a.qf[qfrag_at<R>(b, a.MT, mt, 4 * g + i, 16 * nt + n16, 0)] = hi;
    a.qf[qfrag_at<R>(b, a.MT, mt, 4 * g + i, 16 * nt + n16, 1)] = lo;
  }
}
template <int R>
__global__ __launch_bounds__(64) void mla_qproj_kernel(MlaQArgs a) {
  qproj_wave<R>(a, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x);
}

// The one-call step's first launch (MAX): workgroups 0 .. B-1 append sequence
// b's new latent row (the arithmetic of the stand-alone append), the others
// run the query projection's waves, qw per workgroup (wave w: M-tile w % MT,
// coordinate tile (w / MT) % (R / 16), sequence w / (MT R / 16)); the rest of
// their waves exit at once.  The two are independent, so one launch replaces
// two.  (Two projection waves per workgroup spread them over about 128
// compute units; sixteen queued their 162 loads each on 16 compute units and
// made the launch slower than the two it replaces.)
constexpr int kMlaPrepWaves = 2;
template <int R, int PARTS>
__global__ __launch_bounds__(R * PARTS) void mla_prep_kernel(AppendArgs ap, MlaQArgs qa, int n_append, int qw) {
  static_assert(R * PARTS == 1024, "one 1024-thread workgroup per appended row");
  __shared__ float s_part[R * PARTS];
  if (int(blockIdx.x) < n_append) {
    append_wide_row<1, 1, R, kMlaDk, PARTS>(ap, 0, 0, blockIdx.x, s_part);
    return;
  }
  if (int(threadIdx.x >> 6) >= qw) return;
  const int w = (int(blockIdx.x) - n_append) * qw + int(threadIdx.x >> 6);
  const int NT = R / 16, per_b = qa.MT * NT;
  const int b = w / per_b, rem = w - b * per_b;
  if (b >= n_append) return;  // the last workgroup's spare waves (B sequences)
  qproj_wave<R>(qa, rem % qa.MT, rem / qa.MT, b, int(threadIdx.x & 63));
}

// MEAN: the group-mean query (1/Hq) sum_h q_h, projected once (linearity:
// its projection is the mean of the heads' projections).  Row 0 of the single
// M-tile holds it; rows 1..15 are zero.
template <int R>
__global__ __launch_bounds__(256) void mla_qproj_mean_kernel(MlaQArgs a) {
  constexpr int PARTS = 256 / R;
  constexpr int PER = kMlaDk / PARTS;
  static_assert(kMlaDk % PARTS == 0, "coordinate split");
  __shared__ float s_qm[kMlaDk];
  __shared__ float s_part[256];
  const int b = blockIdx.y;
  const float inv = 1.f / float(a.Hq);
  for (int j = threadIdx.x; j < kMlaDk; j += 256) {
    float s = 0.f;
    for (int h = 0; h < a.Hq; ++h) s += bf16_to_f32(a.q[(size_t(b) * a.Hq + h) * kMlaDk + j]);
    s_qm[j] = s * inv;
  }
  __syncthreads();
  const int r = threadIdx.x % R, part = threadIdx.x / R;
  float acc = 0.f;
  for (int j = part * PER; j < (part + 1) * PER; ++j) acc = fmaf(s_qm[j], a.P[j * R + r], acc);
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * R; i += 256) {
    const int m = i / R, rr = i % R;
    float v = 0.f;
    if (m == 0)
      for (int p = 0; p < PARTS; ++p) v += s_part[p * R + rr];
    uint16_t hi, lo;
    split_bf16(v, &hi, &lo);
    a.qf[qfrag_at<R>(b, 1, 0, m, rr, 0)] = hi;
    a.qf[qfrag_at<R>(b, 1, 0, m, rr, 1)] = lo;
  }
}

// =====================================================================================
// Score scan.  One workgroup per kMlaScoreTile candidate tokens of a sequence,
// in steps of 64 tokens.  The step's projected keys (64 x R bf16) are loaded
// cooperatively with 16-byte loads, kept PF steps ahead in registers, and
// staged in shared memory (16-byte units XOR-swizzled within each 128-byte
// line, so the B-fragment reads are free of bank conflicts).  MAX: wave w
// multiplies the keys with its MTW M-tiles of projected queries (heads
// 64 w .. 64 w + 16 MTW - 1) and keeps the per-token maximum; the four waves'
// maxima are merged through shared memory.  MEAN: wave w scores tokens
// 16 w .. 16 w + 15 of the step against the mean query.  Optionally builds
// the first radix-digit histogram of the scores for selection.
// =====================================================================================
struct MlaScoreArgs {
  const uint16_t* qf;
  const void* kp;         // [B][t_max][R] bf16
  const int32_t* seq_lens;
  float* scores;          // [B][t_max]
  uint32_t* hist1;        // null: no histogram
  uint32_t* row_state;
  int t_max, topk, window, MT;
};

template <int R, int MTW, bool MEAN>
__global__ __launch_bounds__(256, 2) void mla_score_kernel(MlaScoreArgs a) {
  constexpr int KS = R / 32;
  constexpr int STEP_B = 64 * R * 2;   // bytes of one step's projected keys
  constexpr int UT = STEP_B / 16 / 256;  // 16-byte units per thread per step
  constexpr int UPT = R / 8;           // 16-byte units per token
  constexpr int PF = 4;                // steps in flight
  constexpr int NM = MEAN ? 1 : MTW;
  static_assert(UT >= 1, "step size");

  __shared__ __align__(16) char s_kp[2][STEP_B];
  __shared__ float s_red[2][4][64];
  __shared__ uint32_t s_hist[kDigit1Bins];
  __shared__ uint32_t s_scan[8];
  __shared__ uint32_t s_out[2];

  const int tile = blockIdx.x, b = blockIdx.y;
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  const int t0 = tile * kMlaScoreTile;
  if (t0 >= n_cand) return;
  const int t_end = min(t0 + kMlaScoreTile, n_cand);
  const int n_steps = (t_end - t0 + 63) >> 6;
  const bool do_hist = a.hist1 != nullptr && a.topk > 0 && a.topk < n_cand;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, n16 = lane & 15;
  const char* kp_row = reinterpret_cast<const char*>(a.kp) + size_t(b) * a.t_max * (R * 2);
  float* srow = a.scores + size_t(b) * a.t_max;

  auto issue = [&](int step, u32x4_t* v) {
#pragma unroll
    for (int k = 0; k < UT; ++k) {
      const int u = int(threadIdx.x) + 256 * k;
      const int tok = min(t0 + step * 64 + u / UPT, t_end - 1);
      v[k] = ld16_nt(kp_row + size_t(tok) * (R * 2) + (u % UPT) * 16);
    }
  };
  auto stash = [&](int buf, const u32x4_t* v) {
#pragma unroll
    for (int k = 0; k < UT; ++k) {
      const int u = int(threadIdx.x) + 256 * k;
      const int line = u >> 3, uil = u & 7;
      *reinterpret_cast<u32x4_t*>(s_kp[buf] + line * 128 + 16 * (uil ^ (line & 7))) = v[k];
    }
  };
  // B fragment: column n = token 16 q + n16 of the step, contraction indices
  // 32 s + 8 g .. +7 (= 16-byte unit 4 s + g of the token's row)
  auto bfrag = [&](int buf, int q, int s) -> u32x4_t {
    const int u = (16 * q + n16) * UPT + 4 * s + g;
    const int line = u >> 3, uil = u & 7;
    return *reinterpret_cast<const u32x4_t*>(s_kp[buf] + line * 128 + 16 * (uil ^ (line & 7)));
  };

  u32x4_t ring[PF][UT];
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < n_steps) issue(p, ring[p]);

  const int mt0 = MEAN ? 0 : wave * MTW;
  u32x4_t afr[NM][KS][2];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
        afr[m][s][sp] = ld16(a.qf + ((((size_t(b) * a.MT + mt0 + m) * KS + s) * 2 + sp) * 64 + lane) * 8);

  if (do_hist)
    for (int i = threadIdx.x; i < kDigit1Bins; i += 256) s_hist[i] = 0u;
  stash(0, ring[0]);
  if (PF < n_steps) issue(PF, ring[0]);
  __syncthreads();

  for (int i0 = 0; i0 < n_steps; i0 += PF) {
#pragma unroll
    for (int pp = 0; pp < PF; ++pp) {
      const int step = i0 + pp;
      if (step >= n_steps) break;
      const int buf = step & 1;
      if constexpr (MEAN) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4_t bb = bfrag(buf, wave, s);
          c = mfma16(afr[0][s][0], bb, c);
          c = mfma16(afr[0][s][1], bb, c);
        }
        if (g == 0) s_red[buf][wave][n16] = c[0];  // row 0: the mean query
      } else {
        float mine = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x4_t bb[KS];
#pragma unroll
          for (int s = 0; s < KS; ++s) bb[s] = bfrag(buf, q, s);
          float best = -INFINITY;
#pragma unroll
          for (int m = 0; m < MTW; ++m) {
            f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              c = mfma16(afr[m][s][0], bb[s], c);
              c = mfma16(afr[m][s][1], bb[s], c);
            }
            best = fmaxf(best, fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3])));
          }
          best = xor32_max(xor16_max(best));
          if (g == q) mine = best;
        }
        s_red[buf][wave][lane] = mine;
      }
      if (step + 1 < n_steps) {
        stash(buf ^ 1, ring[(pp + 1) % PF]);
        if (step + 1 + PF < n_steps) issue(step + 1 + PF, ring[(pp + 1) % PF]);
      }
      __syncthreads();
      if (wave == (step & 3)) {  // the step's 64 scores (and histogram counts)
        float v;
        if constexpr (MEAN) {
          v = s_red[buf][lane >> 4][lane & 15];
        } else {
          v = fmaxf(fmaxf(s_red[buf][0][lane], s_red[buf][1][lane]),
                    fmaxf(s_red[buf][2][lane], s_red[buf][3][lane]));
        }
        const int t = t0 + step * 64 + lane;
        if (t < t_end) {
          srow[t] = v;
          if (do_hist) atomicAdd(&s_hist[score_key(v) >> (32 - kDigit1Bits)], 1u);
        }
      }
    }
  }

  if (!do_hist) return;
  __syncthreads();
  uint32_t* g_hist = a.hist1 + size_t(b) * kDigit1Bins;
  for (int i = threadIdx.x; i < kDigit1Bins; i += 256) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(&g_hist[i], c);
  }
  uint32_t* g_state = a.row_state + size_t(b) * kRowStateWords;
  const uint32_t n_tiles = uint32_t((n_cand + kMlaScoreTile - 1) / kMlaScoreTile);
  if (!last_arrival(&g_state[RS_TICKET_SCORE], n_tiles)) return;
  finish_first_digit(g_hist, g_state, s_hist, s_scan, s_out, uint32_t(a.topk));
}

// =====================================================================================
// Attention over the selected latent rows.  One workgroup per (sequence, group
// of 32 query heads, chunk of the index list), in sub-blocks of 64 rows.  The
// head group's queries and the chunk's row indices are staged in shared
// memory once; the rows of sub-block j + 1 are loaded into registers while
// sub-block j is processed:
//
//  1. wave w holds rows 16 w .. 16 w + 15 of the sub-block (576 elements each)
//     as A operands and computes S^T (16 rows x 32 heads) against the queries
//     (B operands read from shared memory);
//  2. the first 512 elements of its rows (the values) are stored row-major in
//     shared memory; the P V products read them back as B operands with the
//     transposing ds_read_b64_tr_b16 (within a 16-lane group, lane i receives
//     column i of the four rows that lanes 4 k + q address);
//  3. per-head maxima are merged through shared memory; every wave forms the
//     base-2 probabilities of its 16 rows, split into bf16 hi + lo, in shared
//     memory;
//  4. wave w accumulates O[32 heads x value columns 128 w .. 128 w + 127] +=
//     P V over the 64 rows, after rescaling by the change of the running max.
//
// The chunk's unnormalised output, running max (base 2) and sum are written
// as partials; mla_combine_kernel merges the chunks of a head.
// =====================================================================================
constexpr int kQStride = kMlaDk * 2 + 16;  // bytes per staged query row
constexpr int kVStride = kMlaDv * 2 + 32;  // bytes per staged value row
constexpr int kPStride = 144;              // bytes per probability row (one head): 64 rows + 16 B pad
constexpr int kMlaMaxChunk = 2048;         // rows per attention chunk at most

struct MlaAttnSmem {
  char q[32 * kQStride];
  char v[64 * kVStride];
  char p[2][32 * kPStride];
  int idx[kMlaMaxChunk];
  float mx[4][32];
  float alpha[32];
};

struct MlaAttnArgs {
  const uint16_t* q;      // [B][Hq][576]
  const uint16_t* kv;     // [B][t_max][576]
  const int32_t* idx;     // [B][idx_stride]  (indexed path)
  const int32_t* n_sel;   // [B]              (indexed path)
  const int32_t* seq_lens;  //                (dense path)
  float* part_o;          // [B][n_chunks][Hq][512]
  float* part_ml;         // [B][n_chunks][Hq][2]
  void* out;
  float* lse;
  int Hq, t_max, idx_stride, chunk, n_chunks, out_dtype;
  float qscale;           // softmax scale * log2(e)
};

template <bool INDEXED>
__device__ __forceinline__ int mla_row_count(const MlaAttnArgs& a, int b) {
  int n = INDEXED ? a.n_sel[b] : a.seq_lens[b];
  const int hi = INDEXED ? a.idx_stride : a.t_max;
  return n < 0 ? 0 : (n > hi ? hi : n);
}

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

// B fragment of P V for value columns n0 .. n0 + 15 and sub-block rows
// 32 ks + 8 g .. + 7 (g = lane / 16): two transposing reads of 4 rows each.
__device__ __forceinline__ u32x4_t vfrag(const char* sv, int ks, int n0) {
  const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15;
  const char* base = sv + (32 * ks + 8 * g + (i >> 2)) * kVStride + (n0 + 4 * (i & 3)) * 2;
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t r0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base)));
  const u32x2_t r1 =
      __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base + 4 * kVStride)));
  return u32x4_t{r0.x, r0.y, r1.x, r1.y};
}

template <bool INDEXED>
__global__ __launch_bounds__(256, 1) void mla_attn_kernel(MlaAttnArgs a) {
  constexpr int KS = kMlaDk / 32;
  __shared__ __align__(16) MlaAttnSmem S;
  const int chunk_id = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int h0 = hg * 32;
  const int n = mla_row_count<INDEXED>(a, b);
  const int c0 = chunk_id * a.chunk;
  const int cnt = c0 < n ? min(a.chunk, n - c0) : 0;
  if (cnt == 0) return;  // never read by the combine
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, n16 = lane & 15;

  // the head group's queries and the chunk's row indices into shared memory
  for (int u = threadIdx.x; u < 32 * (kMlaDk / 8); u += 256) {
    const int hh = u / (kMlaDk / 8), c = u - hh * (kMlaDk / 8);
    *reinterpret_cast<u32x4_t*>(S.q + hh * kQStride + c * 16) =
        ld16(a.q + (size_t(b) * a.Hq + h0 + hh) * kMlaDk + c * 8);
  }
  if constexpr (INDEXED) {  // (the dense path's rows are c0 + p)
    for (int i = threadIdx.x; i < cnt; i += 256) {
      const int t = a.idx[size_t(b) * a.idx_stride + c0 + i];
      S.idx[i] = t < 0 ? 0 : (t >= a.t_max ? a.t_max - 1 : t);
    }
  }
  __syncthreads();

  const uint16_t* kvb = a.kv + size_t(b) * a.t_max * kMlaDk;
  // rows: A operand; row m = row 16 wave + n16 of the sub-block.  Plain
  // (temporal) loads: the four head groups of a chunk run on one XCD and read
  // the same rows, so three of the four find them in its L2 (non-temporal
  // loads, which do not keep them there, made the launch about 4 us slower).
  auto load_rows = [&](int sb, u32x4_t (&kf)[KS]) {
    const int p = min(sb * 64 + 16 * wave + n16, cnt - 1);
    const int t = INDEXED ? S.idx[p] : c0 + p;
    const uint16_t* row = kvb + size_t(t) * kMlaDk + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = ld16(row + 32 * s);
  };

  f32x4_t acc[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const int n_sub = (cnt + 63) >> 6;
  const int tau = 16 * wave + n16;  // this lane's row within the sub-block (A layout)

  // kf: this sub-block's rows; kn, loaded here for sub-block `next` once kf's
  // products are issued, stays in flight through the rest of the step
  auto step = [&](int sb, const u32x4_t (&kf)[KS], int next, u32x4_t (&kn)[KS]) {
    f32x4_t st[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    constexpr int QB = 3;  // K-steps whose query fragments are read together
#pragma unroll
    for (int s0 = 0; s0 < KS; s0 += QB) {
      u32x4_t qb[QB][2];
#pragma unroll
      for (int u = 0; u < QB; ++u)
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) qb[u][ht] = ld16(S.q + (16 * ht + n16) * kQStride + (32 * (s0 + u) + 8 * g) * 2);
#pragma unroll
      for (int u = 0; u < QB; ++u)
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) st[ht] = mfma16(kf[s0 + u], qb[u][ht], st[ht]);
    }
    if (next < n_sub) load_rows(next, kn);
    __syncthreads();  // the previous sub-block's readers of v, p and alpha are done
#pragma unroll
    for (int s = 0; s < kMlaDv / 32; ++s)
      *reinterpret_cast<u32x4_t*>(S.v + tau * kVStride + (32 * s + 8 * g) * 2) = kf[s];
    // logits in base 2; result lane holds head 16 ht + n16, rows 16 wave + 4 g + i
    const int pbase = sb * 64 + 16 * wave + 4 * g;
    float x[2][4];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[ht][i] = (pbase + i < cnt) ? st[ht][i] * a.qscale : -INFINITY;
      float mw = fmaxf(fmaxf(x[ht][0], x[ht][1]), fmaxf(x[ht][2], x[ht][3]));
      mw = xor32_max(xor16_max(mw));
      if (g == 0) S.mx[wave][16 * ht + n16] = mw;
    }
    __syncthreads();

    float alpha[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int hh = 16 * ht + n16;
      const float mb = fmaxf(fmaxf(S.mx[0][hh], S.mx[1][hh]), fmaxf(S.mx[2][hh], S.mx[3][hh]));
      const float m_new = fmaxf(m_run[ht], mb);
      alpha[ht] = mla_exp2(m_run[ht] - m_new);
      uint32_t w01[2], w23[2];
      split_bf16x2_terms<2>(mla_exp2(x[ht][0] - m_new), mla_exp2(x[ht][1] - m_new), w01);
      split_bf16x2_terms<2>(mla_exp2(x[ht][2] - m_new), mla_exp2(x[ht][3] - m_new), w23);
      const int off = hh * kPStride + (16 * wave + 4 * g) * 2;
      *reinterpret_cast<uint2*>(S.p[0] + off) = make_uint2(w01[0], w23[0]);
      *reinterpret_cast<uint2*>(S.p[1] + off) = make_uint2(w01[1], w23[1]);
      if (wave == 0 && g == 0) S.alpha[hh] = alpha[ht];
      m_run[ht] = m_new;
    }
    __syncthreads();

    // P as A operand: row m = head 16 mt + n16, contraction = rows 32 ks + 8 g .. +7
    u32x4_t pa[2][2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float rs = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          pa[mt][ks][sp] = ld16(S.p[sp] + (16 * mt + n16) * kPStride + (32 * ks + 8 * g) * 2);
#pragma unroll
          for (int e = 0; e < 4; ++e) rs += bf16_lo(pa[mt][ks][sp][e]) + bf16_hi(pa[mt][ks][sp][e]);
        }
      rs = xor32_add(xor16_add(rs));
      l_run[mt] = fmaf(alpha[mt], l_run[mt], rs);
      // accumulator rows are heads 16 mt + 4 g + i
      const float4 al = *reinterpret_cast<const float4*>(&S.alpha[16 * mt + 4 * g]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        acc[mt][nt][0] *= al.x;
        acc[mt][nt][1] *= al.y;
        acc[mt][nt][2] *= al.z;
        acc[mt][nt][3] *= al.w;
      }
    }
    constexpr int VB = 4;  // value tiles whose fragments are read together
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nt0 = 0; nt0 < 8; nt0 += VB) {
        u32x4_t vb[VB];
#pragma unroll
        for (int u = 0; u < VB; ++u) vb[u] = vfrag(S.v, ks, 128 * wave + 16 * (nt0 + u));
#pragma unroll
        for (int u = 0; u < VB; ++u)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            acc[mt][nt0 + u] = mfma16(pa[mt][ks][0], vb[u], acc[mt][nt0 + u]);
            acc[mt][nt0 + u] = mfma16(pa[mt][ks][1], vb[u], acc[mt][nt0 + u]);
          }
      }
  };

  // sub-blocks in pairs, so that the two row buffers are named statically
  u32x4_t k0[KS], k1[KS];
  load_rows(0, k0);
  for (int sb = 0; sb < n_sub; sb += 2) {
    step(sb, k0, sb + 1, k1);
    if (sb + 1 < n_sub) step(sb + 1, k1, sb + 2, k0);
  }

  const size_t slot = size_t(b) * a.n_chunks + chunk_id;
  float* po = a.part_o + (slot * a.Hq + h0) * kMlaDv;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        po[size_t(16 * mt + 4 * g + i) * kMlaDv + 128 * wave + 16 * nt + n16] = acc[mt][nt][i];
  if (wave == 0 && g == 0) {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float* pml = a.part_ml + (slot * a.Hq + h0 + 16 * ht + n16) * 2;
      pml[0] = m_run[ht];
      pml[1] = l_run[ht];
    }
  }
}

// Log-sum-exp merge of the chunk partials of one (sequence, head), in chunk
// order; out = 0 and lse = -inf when the sequence attends over nothing.  The
// partials are read in batches of kMlaMergeBatch chunks with every load of a
// batch issued at once (chunks past the live count re-read the last live one
// and carry weight 0), and each batch is folded into a running (M, L, o).
constexpr int kMlaMergeBatch = 16;
template <bool INDEXED>
__global__ __launch_bounds__(128) void mla_combine_kernel(MlaAttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int n = mla_row_count<INDEXED>(a, b);
  const int n_live = (n + a.chunk - 1) / a.chunk;
  const size_t oi = (size_t(b) * a.Hq + h) * kMlaDv + 4 * threadIdx.x;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (n_live > 0) {
    const float* ml = a.part_ml + (size_t(b) * a.n_chunks * a.Hq + h) * 2;
    const size_t cstride = size_t(a.Hq) * 2;
    const float* po = a.part_o + (size_t(b) * a.n_chunks * a.Hq + h) * kMlaDv + 4 * threadIdx.x;
    float M = -INFINITY, L = 0.f;
    for (int c0 = 0; c0 < n_live; c0 += kMlaMergeBatch) {
      float m[kMlaMergeBatch], l[kMlaMergeBatch];
      float4 v[kMlaMergeBatch];
#pragma unroll
      for (int i = 0; i < kMlaMergeBatch; ++i) {
        const int c = min(c0 + i, n_live - 1);
        m[i] = ml[c * cstride];
        l[i] = ml[c * cstride + 1];
        v[i] = *reinterpret_cast<const float4*>(po + size_t(c) * a.Hq * kMlaDv);
      }
      float Mb = M;
#pragma unroll
      for (int i = 0; i < kMlaMergeBatch; ++i) Mb = c0 + i < n_live ? fmaxf(Mb, m[i]) : Mb;
      const float sc = (M == -INFINITY) ? 0.f : mla_exp2(M - Mb);
      L *= sc;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] *= sc;
#pragma unroll
      for (int i = 0; i < kMlaMergeBatch; ++i) {
        const float w = (c0 + i < n_live) ? mla_exp2(m[i] - Mb) : 0.f;
        L = fmaf(w, l[i], L);
        o[0] = fmaf(w, v[i].x, o[0]);
        o[1] = fmaf(w, v[i].y, o[1]);
        o[2] = fmaf(w, v[i].z, o[2]);
        o[3] = fmaf(w, v[i].w, o[3]);
      }
      M = Mb;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] /= L;
    lse = (M + __log2f(L)) * kLn2;
  }
  if (a.out_dtype == JSSA_BF16) {
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + oi;
    *reinterpret_cast<uint2*>(out) =
        make_uint2(uint32_t(f32_to_bf16_rne(o[0])) | (uint32_t(f32_to_bf16_rne(o[1])) << 16),
                   uint32_t(f32_to_bf16_rne(o[2])) | (uint32_t(f32_to_bf16_rne(o[3])) << 16));
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) = make_float4(o[0], o[1], o[2], o[3]);
  }
  if (a.lse && threadIdx.x == 0) a.lse[size_t(b) * a.Hq + h] = lse;
}

// ---- launchers -----------------------------------------------------------------------------
static MlaQArgs qproj_args(const jssa_desc& d, const void* q, const float* P, char* ws_base, const Workspace& ws) {
  MlaQArgs qa;
  qa.q = reinterpret_cast<const uint16_t*>(q);
  qa.P = P;
  qa.qf = reinterpret_cast<uint16_t*>(ws_base + ws.qfrag);
  qa.Hq = d.n_q_heads;
  qa.MT = d.reduce == JSSA_REDUCE_MEAN ? 1 : d.n_q_heads / 16;
  return qa;
}

hipError_t launch_mla_qproj(const jssa_desc& d, const void* q, const float* P, char* ws_base, const Workspace& ws,
                            hipStream_t s) {
  const MlaQArgs qa = qproj_args(d, q, P, ws_base, ws);
  const bool mean = d.reduce == JSSA_REDUCE_MEAN;
  if (d.rank == 64) {
    if (mean) hipLaunchKernelGGL(mla_qproj_mean_kernel<64>, dim3(1, d.batch), dim3(256), 0, s, qa);
    else hipLaunchKernelGGL(mla_qproj_kernel<64>, dim3(d.n_q_heads / 16, 4, d.batch), dim3(64), 0, s, qa);
  } else {
    if (mean) hipLaunchKernelGGL(mla_qproj_mean_kernel<32>, dim3(1, d.batch), dim3(256), 0, s, qa);
    else hipLaunchKernelGGL(mla_qproj_kernel<32>, dim3(d.n_q_heads / 16, 2, d.batch), dim3(64), 0, s, qa);
  }
  return hipGetLastError();
}

// The step's new latent rows and the query projection in one launch (MAX
// reduction, bf16 rows, one new row per sequence); false when the shape takes
// the separate launches.
bool mla_prep_fusable(const jssa_desc& d) {
  return d.layout == JSSA_LAYOUT_MLA && d.reduce == JSSA_REDUCE_MAX && d.kv_dtype == JSSA_BF16 &&
         d.kp_dtype == JSSA_BF16 && d.d_k == kMlaDk && d.n_kv_heads == 1 && (d.rank == 64 || d.rank == 32);
}
hipError_t launch_mla_prep(const jssa_desc& d, const void* k_new, const int32_t* pos, const float* P,
                           void* k_cache, void* kp_cache, const void* q, char* ws_base, const Workspace& ws,
                           hipStream_t s) {
  if (!mla_prep_fusable(d)) return hipErrorInvalidValue;
  AppendArgs ap;
  ap.k_new = k_new; ap.v_new = nullptr; ap.pos = pos; ap.P = P;
  ap.k_cache = k_cache; ap.v_cache = nullptr; ap.kp = kp_cache;
  ap.n_new = 1; ap.Hkv = 1; ap.d_k = d.d_k; ap.d_v = d.d_v; ap.t_max = d.t_max; ap.mla = 1;
  const MlaQArgs qa = qproj_args(d, q, P, ws_base, ws);
  const int q_waves = d.batch * qa.MT * (d.rank / 16);
  const int qw = kMlaPrepWaves;
  const dim3 grid(unsigned(d.batch + (q_waves + qw - 1) / qw));
  if (d.rank == 64) hipLaunchKernelGGL((mla_prep_kernel<64, 16>), grid, dim3(1024), 0, s, ap, qa, d.batch, qw);
  else hipLaunchKernelGGL((mla_prep_kernel<32, 32>), grid, dim3(1024), 0, s, ap, qa, d.batch, qw);
  return hipGetLastError();
}

hipError_t launch_mla_scan(const jssa_desc& d, const void* kp, const int32_t* seq_lens, float* scores, bool hist,
                           char* ws_base, const Workspace& ws, hipStream_t s, void* const* ev) {
  const bool mean = d.reduce == JSSA_REDUCE_MEAN;
  MlaScoreArgs sa;
  sa.qf = reinterpret_cast<const uint16_t*>(ws_base + ws.qfrag);
  sa.kp = kp; sa.seq_lens = seq_lens; sa.scores = scores;
  sa.hist1 = hist ? reinterpret_cast<uint32_t*>(ws_base + ws.hist1) : nullptr;
  sa.row_state = hist ? reinterpret_cast<uint32_t*>(ws_base + ws.row_state) : nullptr;
  sa.t_max = d.t_max; sa.topk = d.topk; sa.window = d.window;
  sa.MT = mean ? 1 : d.n_q_heads / 16;
  const dim3 grid((d.t_max + kMlaScoreTile - 1) / kMlaScoreTile, d.batch);
  const bool two = d.n_q_heads / 64 == 2;
  // with `ev`, events ev[0] / ev[1] take the kernel's own start and end
  auto go = [&](auto kernel) {
    if (ev)
      hipExtLaunchKernelGGL(kernel, grid, dim3(256), 0, s, static_cast<hipEvent_t>(ev[0]),
                            static_cast<hipEvent_t>(ev[1]), 0u, sa);
    else
      hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, sa);
  };
  if (d.rank == 64) {
    if (mean) go(mla_score_kernel<64, 1, true>);
    else if (two) go(mla_score_kernel<64, 2, false>);
    else go(mla_score_kernel<64, 1, false>);
  } else {
    if (mean) go(mla_score_kernel<32, 1, true>);
    else if (two) go(mla_score_kernel<32, 2, false>);
    else go(mla_score_kernel<32, 1, false>);
  }
  return hipGetLastError();
}

hipError_t launch_mla_attend(const jssa_desc& d, const void* q, const void* k_cache, const int32_t* idx,
                             const int32_t* n_sel, const int32_t* seq_lens, void* out, float* lse,
                             char* ws_base, const Workspace& ws, hipStream_t s) {
  MlaAttnArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.kv = reinterpret_cast<const uint16_t*>(k_cache);
  a.idx = idx; a.n_sel = n_sel; a.seq_lens = seq_lens;
  a.part_o = reinterpret_cast<float*>(ws_base + ws.part_acc);
  a.part_ml = reinterpret_cast<float*>(ws_base + ws.part_ml);
  a.out = out; a.lse = lse;
  a.Hq = d.n_q_heads; a.t_max = d.t_max; a.idx_stride = d.topk + d.window;
  a.chunk = ws.chunk; a.n_chunks = ws.n_chunks; a.out_dtype = d.out_dtype;
  a.qscale = d.scale * kLog2e;
  if (idx && ws.chunk > kMlaMaxChunk) return hipErrorInvalidValue;  // the chunk's indices are staged
  const dim3 grid(ws.n_chunks, d.n_q_heads / 32, d.batch), cgrid(d.n_q_heads, d.batch);
  if (idx) {
    hipLaunchKernelGGL(mla_attn_kernel<true>, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(mla_combine_kernel<true>, cgrid, dim3(128), 0, s, a);
  } else {
    hipLaunchKernelGGL(mla_attn_kernel<false>, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(mla_combine_kernel<false>, cgrid, dim3(128), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace jssa
