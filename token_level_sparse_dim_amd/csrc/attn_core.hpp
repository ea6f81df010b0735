// Attention core shared by the stand-alone attention launch (attn.hip) and the
// fused decode pipeline (pipeline.hip): one chunk of one (sequence, KV head)
// row, with an online-softmax state per chunk and a log-sum-exp combine by the
// row's last chunk (JSSA summary section 3.3: every selected K/V row is read in
// place once and used by all G query heads of its KV head).
#pragma once

#include "jssa_device.hpp"
#include "jssa_internal.hpp"
#include "resolve.hpp"

namespace jssa {

constexpr int kMaxIdxChunk = 1024;
constexpr int kCombineBatch = 64;  // chunks whose merge weights are staged together
constexpr uint32_t kSpinLimit = 1u << 26;  // bounded wait (seconds): a broken invariant cannot hang

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int32_t* idx;  // input list (indexed attention) or the output list (after a resolve)
  const int32_t* n_sel;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  float* part_acc;
  float* part_ml;
  uint32_t* row_state;
  uint32_t* queue;
  int Hq, Hkv, t_max, idx_stride, chunk, n_chunks, out_dtype;
  int n_resolve, n_items, attend;
  float qscale;  // softmax scale * log2(e): logits are kept in base 2
  ResolveArgs res;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int G, int D, bool INDEXED, bool RESOLVE>
struct AttnSmem {
  static_assert(4 * G * D >= kCombineBatch * G + 2 * G, "combine scratch fits in acc");
  int idx[INDEXED ? kMaxIdxChunk : 1];
  float m[4][G], l[4][G];
  float acc[4][G][D];
  uint32_t tab[RESOLVE ? 2 * kMaxSelTiles : 1];  // tile tables of extract_range
  uint32_t scan[8];
};

// The last workgroup of the launch resets the queue for the next call.
__device__ __forceinline__ void finish_item(const AttnArgs& a) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t done = __hip_atomic_fetch_add(&a.queue[QW_DONE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == uint32_t(a.n_items) - 1u) {
      __hip_atomic_store(&a.queue[QW_NEXT], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.queue[QW_DONE], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The last chunk of a row to finish: log-sum-exp merge of the row's non-empty
// chunk partials (in chunk order) into out (and lse), or out = 0, lse = -inf
// when the row attends over nothing.  Two rounds of loads: one wave per head
// reads every chunk's (max, sum) at once and forms the head's global max M,
// the chunk weights exp2(m_c - M) and the total L; then every thread reads the
// partial outputs of its elements for all chunks of a batch at once.  sw:
// shared scratch of kCombineBatch * G + 2 * G floats, free at this point.

template <int D, int G>
__device__ __forceinline__ void combine_chunks(const AttnArgs& a, int row, int b, int h, int n, float* sw) {
  const int n_live = (n + a.chunk - 1) / a.chunk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int PER = (G * D + 255) / 256;  // output elements per thread
  if (n_live == 0) {  // nothing attended: out = 0, lse = -inf
    for (int j = threadIdx.x; j < G * D; j += 256) {
      const size_t o = (size_t(b) * a.Hq + size_t(h) * G) * D + j;
      if (a.out_dtype == JSSA_BF16) reinterpret_cast<uint16_t*>(a.out)[o] = 0;
      else reinterpret_cast<float*>(a.out)[o] = 0.f;
    }
    if (a.lse && threadIdx.x < G) a.lse[size_t(b) * a.Hq + h * G + threadIdx.x] = -INFINITY;
    return;
  }
  const float* racc = a.part_acc + size_t(row) * a.n_chunks * G * D;
  const float* rml = a.part_ml + size_t(row) * a.n_chunks * G * 2;
  float* sM = sw;
  float* sL = sw + G;
  float* sW = sw + 2 * G;  // [kCombineBatch][G]
  // global max of each head
  for (int g = wave; g < G; g += 4) {
    float M = -INFINITY;
    for (int c = lane; c < n_live; c += 64) M = fmaxf(M, consume(&rml[(c * G + g) * 2]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (lane == 0) {
      sM[g] = M;
      sL[g] = 0.f;
    }
  }
  __syncthreads();
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  for (int cb = 0; cb < n_live; cb += kCombineBatch) {
    const int nb = min(kCombineBatch, n_live - cb);
    for (int g = wave; g < G; g += 4) {
      float lw = 0.f;
      if (lane < nb) {
        const int c = cb + lane;
        const float m = consume(&rml[(c * G + g) * 2]), l = consume(&rml[(c * G + g) * 2 + 1]);
        const float w = (m == -INFINITY) ? 0.f : fast_exp2(m - sM[g]);
        sW[lane * G + g] = w;
        lw = w * l;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) lw += __shfl_xor(lw, off);
      if (lane == 0) sL[g] += lw;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = k * 256 + int(threadIdx.x);
      if (j < G * D) {
        const int g = j / D;
        float v[kCombineBatch];
#pragma unroll
        for (int c = 0; c < kCombineBatch; ++c) v[c] = c < nb ? consume(&racc[size_t(cb + c) * G * D + j]) : 0.f;
#pragma unroll
        for (int c = 0; c < kCombineBatch; ++c)
          if (c < nb) acc[k] = fmaf(sW[c * G + g], v[c], acc[k]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int j = k * 256 + int(threadIdx.x);
    if (j >= G * D) continue;
    const int g = j / D, dd = j - g * D;
    const float o = acc[k] / sL[g];
    const size_t oi = (size_t(b) * a.Hq + size_t(h) * G + g) * D + dd;
    if (a.out_dtype == JSSA_BF16) reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(o);
    else reinterpret_cast<float*>(a.out)[oi] = o;
    if (dd == 0 && a.lse) a.lse[size_t(b) * a.Hq + h * G + g] = (sM[g] + __log2f(sL[g])) * kLn2;
  }
}

// One chunk of one row: positions [chunk_id*chunk, ...) of the row's n
// tokens; for the indexed path their token indices are already in S.idx.
// RESET_READY: the row's last chunk also clears the row's ready flag (the
// chunks waited for it).  Smem provides idx[], m[4][G], l[4][G], acc[4][G][D].
// Returns true in the one workgroup of the row that merged the chunks.
template <int KVT, int D, int G, bool INDEXED, bool RESET_READY, int U = JSSA_ATTN_UNROLL, typename Smem>
__device__ bool attend_chunk(const AttnArgs& a, Smem& S, int row, int b, int h, int chunk_id, int n) {
  constexpr int EB = Elem<KVT>::bytes;
  constexpr int EPL = Elem<KVT>::per16;
  constexpr int LR = D / EPL;   // lanes per K/V row
  constexpr int RPW = 64 / LR;  // rows per wave per load
  constexpr int NS = 4 * RPW;   // token streams per workgroup
  // U: tokens per stream per step
  static_assert(LR >= 4 && LR <= 32, "row split");

  const int c0 = chunk_id * a.chunk;
  const int cnt = c0 < n ? min(c0 + a.chunk, n) - c0 : 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* pacc = a.part_acc + (size_t(row) * a.n_chunks + chunk_id) * G * D;
  float* pml = a.part_ml + (size_t(row) * a.n_chunks + chunk_id) * G * 2;

  if (cnt > 0) {
    const int p = lane % LR, sidx = wave * RPW + lane / LR;
    float qreg[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 raw = load16(reinterpret_cast<const char*>(a.q) +
                               ((size_t(b) * a.Hq + size_t(h) * G + g) * D + p * EPL) * EB);
      float tmp[EPL];
      unpack16<KVT>(raw, tmp);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qreg[g][e] = tmp[e] * a.qscale;
    }
    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }
    const char* kbase = reinterpret_cast<const char*>(a.k);
    const char* vbase = reinterpret_cast<const char*>(a.v);
    const size_t row_stride = size_t(a.Hkv) * D * EB;  // bytes between consecutive tokens
    const size_t head_off = (size_t(b) * a.t_max * a.Hkv + h) * D * EB + size_t(p) * EPL * EB;
    // K/V loads carry no per-lane branch (past-the-end streams re-read a valid
    // row and are masked out), so the next step's rows stay in flight while the
    // current ones are used.
    auto row_off = [&](int i) {
      const int ic = min(i, cnt - 1);
      const int t = INDEXED ? min(max(S.idx[ic], 0), a.t_max - 1) : c0 + ic;  // indices are clamped
      return head_off + size_t(t) * row_stride;
    };
    uint4 kn[U], vn[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t off = row_off(u * NS + sidx);
      kn[u] = load16_nt(kbase + off);
      vn[u] = load16_nt(vbase + off);
    }
    for (int i0 = 0; i0 < cnt; i0 += NS * U) {
      uint4 kr[U], vr[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = kn[u];
        vr[u] = vn[u];
        valid[u] = i0 + u * NS + sidx < cnt;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t off = row_off(i0 + NS * U + u * NS + sidx);
        kn[u] = load16_nt(kbase + off);
        vn[u] = load16_nt(vbase + off);
      }
      float lg[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kf[EPL];
        unpack16<KVT>(kr[u], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) s = fmaf(qreg[g][e], kf[e], s);
          s = group_sum<LR>(s);
          lg[u][g] = valid[u] ? s : -INFINITY;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = lg[0][g];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, lg[u][g]);
        const float mnew = fmaxf(m[g], mx);
        if (mnew == -INFINITY) continue;
        const float alpha = fast_exp2(m[g] - mnew);
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
        m[g] = mnew;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float pu = fast_exp2(lg[u][g] - mnew);
          l[g] += pu;
          float vf[EPL];
          unpack16<KVT>(vr[u], vf);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pu, vf[e], acc[g][e]);
        }
      }
    }
    // merge the RPW streams of each wave (rows LR lanes apart)
#pragma unroll
    for (int off = LR; off < 64; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mo = __shfl_xor(m[g], off);
        const float lo = __shfl_xor(l[g], off);
        const float M = fmaxf(m[g], mo);
        const float a1 = (m[g] == -INFINITY) ? 0.f : fast_exp2(m[g] - M);
        const float a2 = (mo == -INFINITY) ? 0.f : fast_exp2(mo - M);
        l[g] = l[g] * a1 + lo * a2;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * a1 + __shfl_xor(acc[g][e], off) * a2;
        m[g] = M;
      }
    }
    if (lane < LR) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (lane == 0) { S.m[wave][g] = m[g]; S.l[wave][g] = l[g]; }
#pragma unroll
        for (int e = 0; e < EPL; ++e) S.acc[wave][g][p * EPL + e] = acc[g][e];
      }
    }
    __syncthreads();
    // merge the 4 waves -> this chunk's partial state, published for the combine
    for (int j = threadIdx.x; j < G * D; j += 256) {
      const int g = j / D, dd = j - g * D;
      float M = S.m[0][g];
#pragma unroll
      for (int w = 1; w < 4; ++w) M = fmaxf(M, S.m[w][g]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = (S.m[w][g] == -INFINITY) ? 0.f : fast_exp2(S.m[w][g] - M);
        L = fmaf(S.l[w][g], sc, L);
        A = fmaf(S.acc[w][g][dd], sc, A);
      }
      publish(&pacc[j], A);
      if (dd == 0) { publish(&pml[2 * g], M); publish(&pml[2 * g + 1], L); }
    }
  }

  // every chunk of the row arrives; the last one combines the non-empty chunks
  uint32_t* rstate = a.row_state + size_t(row) * kRowStateWords;
  if (!last_arrival(&rstate[RS_TICKET_ATTN], uint32_t(a.n_chunks))) return false;
  if (RESET_READY && threadIdx.x == 0) publish(&rstate[RS_READY], 0u);  // every chunk has passed its wait
  combine_chunks<D, G>(a, row, b, h, n, &S.acc[0][0][0]);
  return true;
}

// Folds a batch of kMergeBatch chunk partials (max m, sum l, value v; chunks
// past the live count carry m = -inf) into a running log-sum-exp (M, L, A).
constexpr int kMergeBatch = 16;

template <int D, int G>
__device__ __forceinline__ void merge_fold(float& M, float& L, float& A, const float (&m)[kMergeBatch],
                                           const float (&l)[kMergeBatch], const float (&v)[kMergeBatch]) {
  float Mb = M;
#pragma unroll
  for (int i = 0; i < kMergeBatch; ++i) Mb = fmaxf(Mb, m[i]);
  const float sc = (M == -INFINITY) ? 0.f : fast_exp2(M - Mb);
  L *= sc;
  A *= sc;
#pragma unroll
  for (int i = 0; i < kMergeBatch; ++i) {
    const float w = (m[i] == -INFINITY) ? 0.f : fast_exp2(m[i] - Mb);
    L = fmaf(w, l[i], L);
    A = fmaf(w, v[i], A);
  }
  M = Mb;
}

// The merge of a row's n_live parts by the last part to finish, in the same
// launch (the partials were published with device-scope stores before the
// ticket): thread j < G * D owns output element j; every part's (m, l, acc) is
// requested in batches of kMergeBatch device-scope loads and folded in part
// order.
template <int D, int G>
__device__ __forceinline__ void merge_row_in_launch(const AttnArgs& a, int row, int n_live) {
  const int j = threadIdx.x;
  if (j >= G * D) return;
  const int b = row / a.Hkv, h = row - b * a.Hkv;
  const int g = j / D, dd = j - g * D;
  const size_t oi = (size_t(b) * a.Hq + size_t(h) * G + g) * D + dd;
  const float* racc = a.part_acc + size_t(row) * a.n_chunks * G * D + size_t(g) * D + dd;
  const float* rml = a.part_ml + size_t(row) * a.n_chunks * G * 2 + size_t(g) * 2;
  float M = -INFINITY, L = 0.f, A = 0.f;
  for (int c0 = 0; c0 < n_live; c0 += kMergeBatch) {
    float m[kMergeBatch], l[kMergeBatch], v[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const bool ok = c0 + i < n_live;
      m[i] = ok ? consume(&rml[size_t(c0 + i) * G * 2]) : -INFINITY;
      l[i] = ok ? consume(&rml[size_t(c0 + i) * G * 2 + 1]) : 0.f;
      v[i] = ok ? consume(&racc[size_t(c0 + i) * G * D]) : 0.f;
    }
    merge_fold<D, G>(M, L, A, m, l, v);
  }
  const float o = n_live > 0 ? A / L : 0.f;
  if (a.out_dtype == JSSA_BF16) reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(o);
  else reinterpret_cast<float*>(a.out)[oi] = o;
  if (dd == 0 && a.lse) a.lse[size_t(b) * a.Hq + h * G + g] = n_live > 0 ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// ---- one row's portion of its index list, by NW waves --------------------------------
// The fused decode's attention: the workgroup that selected a row's tokens (or
// read them from a caller's list) attends over its portion of the list, `cnt`
// token indices in sidx[].  Sub-chunks of CH = NW * RPW * NL tokens: the K
// and V rows of a sub-chunk are requested with NL 16-byte loads of each per
// lane (lane (p, rsub) taking elements EPL p .. EPL p + EPL - 1 of rows rsub,
// rsub + RPW, ...); the next sub-chunk's K rows as soon as this one's logits
// are formed, its V rows as soon as this one's values are weighed.  (The
// dense decode runs the same portions over every position.)
// Per sub-chunk:
//   pass 1: the G heads' logits -> shared memory (bf16: v_dot2c_f32_bf16 on
//           the packed bf16 pairs of K and of the unscaled query, products
//           exact and summed in fp32, then scaled; fp32: fma chains with the
//           scaled query);
//   one wave per head: the sub-chunk's max against the running max M, the
//           weights exp2(logit - M'), their sum added to the running sum L
//           after scaling it by exp2(M - M');
//   pass 2: every lane scales its running V sums by the same factor and adds
//           its rows' weighted V.
// At the end the row groups of each wave are summed through lane swaps and
// the NW waves through shared memory, and the portion's partial (M, L, acc)
// is written with device-scope stores for the merge by the row's last part
// (merge_row_in_launch).
template <int KVT, int D, int NW, int NL>
struct PortionShape {
  static constexpr int EB = Elem<KVT>::bytes;
  static constexpr int EPL = Elem<KVT>::per16;
  static constexpr int LR = D / EPL;   // lanes per K/V row
  static constexpr int RPW = 64 / LR;  // rows per wave per load
  static constexpr int CH = NW * RPW * NL;
};

template <int KVT, int D, int G, int NW, int NL>
struct PortionSmem {
  static constexpr int CH = PortionShape<KVT, D, NW, NL>::CH;
  // the group's queries: bf16 as stored (packed pairs), fp32 scaled to base-2 logits
  alignas(16) uint32_t q[KVT == 1 ? G * D / 2 : G * D];
  alignas(16) float w[CH][G];  // logits, then weights
  float ml[G][4];              // running max M, running sum L, this sub-chunk's rescale factor
  float acc[NW][G][D];         // per-wave partial outputs
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The group's queries in S.q: bf16 as stored, in 16-byte pieces (thread i
// < G D / 8 holds piece i of the G rows); fp32 one element per thread (i < G
// D), scaled to base-2 logits.  Requested here with the first sub-chunk's
// K/V rows, so their latencies overlap.
template <int KVT, int D, int G>
__device__ __forceinline__ uint4 load_query_piece(const AttnArgs& a, int b, int h) {
  constexpr int NP = KVT == 1 ? G * D / 8 : G * D;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  const size_t q0 = (size_t(b) * a.Hq + size_t(h) * G) * D;
  if (threadIdx.x < NP) {
    if constexpr (KVT == 1) v = load16(reinterpret_cast<const uint16_t*>(a.q) + q0 + threadIdx.x * 8);
    else v.x = __float_as_uint(reinterpret_cast<const float*>(a.q)[q0 + threadIdx.x] * a.qscale);
  }
  return v;
}

template <int KVT, int D, int G, int NW, int NL, bool PUBLISH = false>
__device__ __forceinline__ void attend_portion(const AttnArgs& a, PortionSmem<KVT, D, G, NW, NL>& S,
                                               const int* sidx, int row, int b, int h, int part, int cnt) {
  using SH = PortionShape<KVT, D, NW, NL>;
  constexpr int EB = SH::EB, EPL = SH::EPL, LR = SH::LR, RPW = SH::RPW, CH = SH::CH;
  constexpr int QW = KVT == 1 ? EPL / 2 : EPL;  // query words per lane and head
  static_assert(LR >= 4 && LR <= 32 && G <= NW, "row split");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane % LR, rsub = lane / LR;
  float* pacc = a.part_acc + (size_t(row) * a.n_chunks + part) * G * D;
  float* pml = a.part_ml + (size_t(row) * a.n_chunks + part) * G * 2;
  if (cnt <= 0) return;  // an empty portion past the row's list: the merge ignores it
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const size_t row_stride = size_t(a.Hkv) * D * EB;
  const size_t head_off = (size_t(b) * a.t_max * a.Hkv + h) * D * EB + size_t(p) * EPL * EB;
  const int n_sub = (cnt + CH - 1) / CH;
  // K or V rows of sub-chunk c (rows past cnt re-read a valid row and get weight 0)
  auto load_rows = [&](int c, const char* base, uint4 (&rr)[NL]) {
    const int c0 = min(c, n_sub - 1) * CH;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int r = (k * NW + wave) * RPW + rsub;
      const int t = min(max(sidx[min(c0 + r, cnt - 1)], 0), a.t_max - 1);  // indices are clamped
      rr[k] = load16_nt(base + head_off + size_t(t) * row_stride);
    }
  };
  const uint4 qpiece = load_query_piece<KVT, D, G>(a, b, h);
  uint4 kA[NL], vA[NL];
  load_rows(0, kbase, kA);
  load_rows(0, vbase, vA);
  constexpr int NQP = KVT == 1 ? G * D / 8 : G * D;
  static_assert(NQP <= NW * 64, "query staging");
  if (threadIdx.x < NQP) {
    if constexpr (KVT == 1) reinterpret_cast<uint4*>(S.q)[threadIdx.x] = qpiece;
    else S.q[threadIdx.x] = qpiece.x;
  }
  if (threadIdx.x < G) {
    S.ml[threadIdx.x][0] = -INFINITY;
    S.ml[threadIdx.x][1] = 0.f;
  }
  __syncthreads();  // S.q staged, S.ml set
  uint32_t qreg[G][QW];
  float acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < QW; ++e) qreg[g][e] = S.q[(g * D + p * EPL) / (EPL / QW) + e];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }
  // pass 1: the sub-chunk's logits into S.w
  auto logits = [&](int c, const uint4 (&kr)[NL]) {
    const int n = min(CH, cnt - c * CH);
    // pass 1: logits
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int r = (k * NW + wave) * RPW + rsub;
      const uint32_t kw[4] = {kr[k].x, kr[k].y, kr[k].z, kr[k].w};
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
        if constexpr (KVT == 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) s = dot2_bf16(kw[e], qreg[g][e], s);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) s = fmaf(__uint_as_float(qreg[g][e]), __uint_as_float(kw[e]), s);
        }
        s = group_sum<LR>(s);
        if (KVT == 1) s *= a.qscale;
        if (p == 0) S.w[r][g] = (r < n) ? s : -INFINITY;
      }
    }
  };
  // the running max and sum per head (one wave per head), this sub-chunk's weights
  auto weights = [&]() {
    __syncthreads();
    if (wave < G) {
      const int g = wave;
      float mx = -INFINITY;
      for (int r = lane; r < CH; r += 64) mx = fmaxf(mx, S.w[r][g]);
      mx = group_max<64>(mx);
      const float m_old = S.ml[g][0];
      const float m_new = fmaxf(m_old, mx);  // finite: the sub-chunk has a valid row
      float sum = 0.f;
      for (int r = lane; r < CH; r += 64) {
        const float x = S.w[r][g];
        const float wgt = (x == -INFINITY) ? 0.f : fast_exp2(x - m_new);
        S.w[r][g] = wgt;
        sum += wgt;
      }
      sum = group_sum<64>(sum);
      if (lane == 0) {
        const float alpha = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - m_new);
        S.ml[g][0] = m_new;
        S.ml[g][1] = S.ml[g][1] * alpha + sum;
        S.ml[g][2] = alpha;
      }
    }
    __syncthreads();
  };
  auto weigh_values = [&](int c, const uint4 (&vr)[NL]) {
    // pass 2: weighted V rows (the running sums rescaled first, after the first sub-chunk)
    if (c > 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float alpha = S.ml[g][2];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
      }
    }
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int r = (k * NW + wave) * RPW + rsub;
      float vf[EPL];
      unpack16<KVT>(vr[k], vf);
      float wr[G];
      if constexpr (G == 4) {  // one 16-byte shared-memory read
        const float4 w4 = *reinterpret_cast<const float4*>(&S.w[r][0]);
        wr[0] = w4.x; wr[1] = w4.y; wr[2] = w4.z; wr[3] = w4.w;
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) wr[g] = S.w[r][g];
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(wr[g], vf[e], acc[g][e]);
    }
    __syncthreads();  // S.w and the factors are rewritten by the next sub-chunk
  };
  // The next sub-chunk's K rows are requested as soon as this one's logits
  // are formed, its V rows as soon as this one's values are weighed: no
  // extra registers, and the waits count the loads in issue order (K then
  // V).  The last sub-chunk is peeled so that nothing is requested past it.
  for (int c = 0; c + 1 < n_sub; ++c) {
    logits(c, kA);
    load_rows(c + 1, kbase, kA);
    weights();
    weigh_values(c, vA);
    load_rows(c + 1, vbase, vA);
  }
  logits(n_sub - 1, kA);
  weights();
  weigh_values(n_sub - 1, vA);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = sum_across_groups<LR>(acc[g][e]);
  if (lane < LR) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) S.acc[wave][g][p * EPL + e] = acc[g][e];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < G * D; j += NW * 64) {
    const int g = j / D, dd = j - g * D;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w += 2) v += S.acc[w][g][dd] + S.acc[w + 1][g][dd];
    if (PUBLISH) {  // read by the row's last part in this launch
      publish(&pacc[j], v);
      if (dd == 0) {
        publish(&pml[2 * g], S.ml[g][0]);
        publish(&pml[2 * g + 1], S.ml[g][1]);
      }
    } else {
      pacc[j] = v;
      if (dd == 0) {
        pml[2 * g] = S.ml[g][0];
        pml[2 * g + 1] = S.ml[g][1];
      }
    }
  }
}

}  // namespace jssa
