// Sparse decode step in two launches (JSSA summary Figure 1 and section E.1:
// subspace score scan, per-KV-head top-k selection, gather-free indexed
// attention).
//
// Scan launch, items in order (workgroup i takes items i, i + grid, ...):
//   SAMPLE(row)     a candidate threshold L for the row from a strided sample
//                   of its scores: a key far enough below the sample's estimate
//                   of the k-th key that, with overwhelming probability, at
//                   least k tokens score >= L.  Rows with nothing to choose
//                   (every candidate taken, or none) get their index list here.
//   SCORE(row, i)   scores run i of the row's tokens, streaming the
//                   projected-key cache once, and writes the tokens scoring
//                   >= L, in token order, to each tile's candidate slot.  Runs
//                   are sized so that one run per resident workgroup covers
//                   the rows: a run streams long enough that its row's
//                   threshold is known by the time it is needed.
// Select + attend launch, a few workgroups per row (the parts of its list):
//   each part finds the exact k-th key and tie cut among the row's candidates
//   (the same selection in every part of the row), keeps its own positions of
//   the ascending index list plus window (writing them to the output list),
//   and attends over them; the row's last part to finish (a ticket) merges
//   the parts' partials with a log-sum-exp combine.  If fewer than k tokens
//   reached L (the sample misled), the row is redone exactly: its scores are
//   recomputed, first for the exact top radix digit of the k-th key, then to
//   rewrite the candidate slots from that digit (every part writes the same
//   values).
// Data passes between launches through plain stores and loads; the only wait
// inside a launch is a score run's on its row's sample (an item of a lower
// workgroup index), bounded in time (the merge takes no wait: the last ticket
// holder reads the others' device-scope partials).
#include <math.h>

#include <type_traits>

#include <hip/hip_ext.h>

#include "attn_core.hpp"
#include "jssa_device.hpp"
#include "jssa_internal.hpp"
#include "score_core.hpp"
#include "select_common.hpp"

namespace jssa {

#ifndef JSSA_PIPE_TILE_TOKENS
#define JSSA_PIPE_TILE_TOKENS 1024
#endif
constexpr int kPipeTileTokens = JSSA_PIPE_TILE_TOKENS;  // tokens per tile (at least two workgroup steps)
constexpr int kPipeSampleTokens = 1024;                 // tokens of the threshold sample
constexpr int kPipePF = 3;             // score-scan steps in flight per workgroup
constexpr int kPipeMaxItem = 8192;     // tokens per score item at most (whole tiles)
constexpr int kPipeCandLds = 16384;    // candidates resolved in shared memory
constexpr int kPipeSampleMin = 8192;   // candidate tokens above which a row's threshold is sampled
// Leaves the remaining rounds of a loop over MAXPER rounds of candidates:
// `break` where the loop still unrolls fully with it (MAXPER <= 8), else
// `continue` (the unroller gives up on the larger loops with a second exit,
// and their register arrays would go to scratch).
#define JSSA_ROUNDS_END \
  if constexpr (MAXPER <= 8) {  \
    break;                      \
  } else {                      \
    continue;                   \
  }
constexpr int kPipeMaxTiles = 2048;    // tiles per row
constexpr int kPipeCutList = 256;      // candidates of the cut's bin ranked directly (one per thread)
constexpr int kPipeGatherTiles = 8;    // tiles per wave per gather round
constexpr int kResolveThreads = 1024;  // threads of a resolve workgroup
#ifndef JSSA_PORTION_NL
#define JSSA_PORTION_NL 2
#endif
constexpr int kPortionNL = JSSA_PORTION_NL;  // K and V row loads per lane per attention sub-chunk
#ifndef JSSA_DENSE_NL
#define JSSA_DENSE_NL 2
#endif
constexpr int kDenseNL = JSSA_DENSE_NL;  // the same for the dense decode's parts
constexpr int kPipeMaxPortion = 2048;  // list positions per select/attend workgroup at most
constexpr int kPipeMaxParts = 16;      // select/attend workgroups per row at most
constexpr int kPipePartTarget = 256;   // select/attend workgroups a launch aims for (one per CU)

// per-row state word of the scan (zero on entry and exit): u64 at words 12-13,
// kLwSet | L once the row's threshold is known, plus kLwAppended once the
// step's new token is in the row's caches (a decode that appends it)
constexpr int PW_L = 12;
constexpr uint64_t kLwSet = uint64_t(1) << 32;
constexpr uint64_t kLwAppended = uint64_t(1) << 33;
#ifndef JSSA_PIPE_PER_CU
#define JSSA_PIPE_PER_CU 3  // scan workgroups per compute unit at most (0: as many as fit)
#endif

struct PipeArgs {
  AttnArgs at;  // q, k, v, idx and n_sel (outputs), seq_lens, out, lse, partials, row_state, queue
  const float* P;
  const void* kp;
  uint64_t* cand;      // [rows][t_max] candidate slots, ts entries per tile
  float* qp_pub;       // [rows][G * r] projected queries, left by the sample for an exact re-selection
  // the step's new token, appended in this launch (k_new == nullptr: already appended)
  const void* k_new;   // [B, 1, Hkv, d] (and v_new), written at t = pos[b]
  const void* v_new;
  const int32_t* pos;
  void* k_w;           // the caches, writable
  void* v_w;
  void* kp_w;
  int attend_only;     // host side: launch the attention and merge only, on caller lists
  uint32_t* tile_cnt;  // [rows][n_tiles]
  int G, d_k, topk, window, q_dtype, ts, n_tiles, n_rows, n_attn;
  int samples_in_scan;  // 1: scan workgroup r < n_rows samples row r; 0: a sample launch ran before the scan
  uint64_t spin_ticks;  // wall-clock ticks after the launch's start when every wait gives up
};

__device__ __forceinline__ void flag_error(const PipeArgs& a) { publish(a.at.queue + QW_ERR, 1u); }

// Waits are bounded in time (a broken invariant ends the launch with the error
// flag set instead of hanging it).
__device__ __forceinline__ bool past(uint64_t deadline) { return wall_clock64() > deadline; }

// One wave: the bin of a 2048-bin histogram that holds the need-th largest
// element, counting from the top; out[0] = the bin, out[1] = the number of
// elements in higher bins (1 <= need <= total).  Lane l sums the 32 bins of
// segment 63 - l (read from a per-lane rotation, so the lanes hit different
// banks); a scan over the lanes finds the segment, whose 32 bins are then
// spread over 32 lanes and scanned again.
__device__ __forceinline__ void top_bin_wave(const uint32_t* hist, uint32_t need, uint32_t* out) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t seg = 63u - lane;
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) sum += hist[seg * 32u + ((uint32_t(j) + lane) & 31u)];
  const uint32_t incl = wave_scan_incl(sum);
  const uint64_t hit = __ballot(incl >= need);
  const uint32_t l_star = hit ? uint32_t(__ffsll(static_cast<long long>(hit)) - 1) : 63u;  // first from the top
  const uint32_t above = uint32_t(__builtin_amdgcn_readlane(int(incl - sum), int(l_star)));
  const uint32_t seg_star = 63u - l_star;
  // lane i < 32: bin seg_star * 32 + 31 - i (descending)
  const uint32_t c = lane < 32u ? hist[seg_star * 32u + 31u - lane] : 0u;
  const uint32_t incl2 = above + wave_scan_incl(c);
  const uint64_t hit2 = __ballot(lane < 32u && incl2 >= need);
  const uint32_t i_star = hit2 ? uint32_t(__ffsll(static_cast<long long>(hit2)) - 1) : 31u;
  if (lane == i_star) {
    out[0] = seg_star * 32u + 31u - i_star;
    out[1] = incl2 - c;
  }
}

// One wave: the bin of a 256-bin histogram that holds the need-th smallest
// element, counting from the bottom; out[0] = the bin, out[1] = the number of
// elements in lower bins (1 <= need <= total).  Lane l holds bins 4l .. 4l + 3.
__device__ __forceinline__ void bottom_bin_wave(const uint32_t* hist, uint32_t need, uint32_t* out) {
  const uint32_t lane = threadIdx.x & 63;
  const uint4 c = reinterpret_cast<const uint4*>(hist)[lane];
  const uint32_t sum = c.x + c.y + c.z + c.w;
  const uint32_t incl = wave_scan_incl(sum);
  const uint64_t hit = __ballot(incl >= need);
  const uint32_t l_star = hit ? uint32_t(__ffsll(static_cast<long long>(hit)) - 1) : 63u;
  if (lane == l_star) {
    uint32_t cum = incl - sum, bin = 4u * lane + 3u;
    if (cum + c.x >= need) bin = 4u * lane;
    else if (cum + c.x + c.y >= need) { bin = 4u * lane + 1u; cum += c.x; }
    else if (cum + c.x + c.y + c.z >= need) { bin = 4u * lane + 2u; cum += c.x + c.y; }
    else cum += c.x + c.y + c.z;
    out[0] = bin;
    out[1] = cum;
  }
}

// The need-th largest key among n candidates ((index << 32) | key, read via
// `get`), with the tie cut: exactly `need` candidates satisfy
// key > K* or (key == K* and index <= I*).  Radix digits of 11, 11 and 10 bits
// over shared-memory histograms (`hist`: 2048 words, 16-byte aligned), each
// digit's bin found by the first wave; ties by the index bits 23..16, 15..8,
// 7..0.  1 <= need <= n; NT threads.
template <int NT, typename Get>
__device__ __forceinline__ void kth_cut(Get get, uint32_t n, uint32_t need, bool want_ties, uint32_t* hist,
                                        uint32_t* out, uint32_t* kstar_out, uint32_t* istar_out) {
  const uint32_t tid = threadIdx.x;
  // one digit: `bin_of` maps a candidate to its bin, or to none (>= 2048)
  auto digit = [&](auto bin_of) {
    for (uint32_t i = tid; i < 2048u; i += NT) hist[i] = 0u;
    __syncthreads();
    for (uint32_t j = tid; j < n; j += NT) {
      const uint32_t d = bin_of(get(j));
      if (d < 2048u) atomicAdd(&hist[d], 1u);
    }
    __syncthreads();
    if (tid < 64) top_bin_wave(hist, need, out);
    __syncthreads();
    const uint32_t bin = out[0];
    need -= out[1];
    return bin;
  };
  // digit A: bits 31..21
  const uint32_t dA = digit([](uint64_t c) { return uint32_t(c) >> 21; });
  __syncthreads();
  // digit B: bits 20..10
  const uint32_t dB = digit([&](uint64_t c) {
    const uint32_t key = uint32_t(c);
    return (key >> 21) == dA ? (key >> 10) & 0x7ffu : 2048u;
  });
  const uint32_t hi22 = (dA << 11) | dB;
  __syncthreads();
  // digit C: bits 9..0
  const uint32_t dC = digit([&](uint64_t c) {
    const uint32_t key = uint32_t(c);
    return (key >> 10) == hi22 ? key & 0x3ffu : 2048u;
  });
  const uint32_t m_ties = need;  // of the keys equal to K*, the m_ties lowest indices are taken
  const uint32_t n_eq = hist[dC];
  const uint32_t kstar = (hi22 << 10) | dC;
  __syncthreads();
  uint32_t istar = 0xffffffffu;
  if (want_ties && m_ties < n_eq) {
    uint32_t prefix = 0, m = m_ties;
    for (int shift = 16; shift >= 0; shift -= 8) {
      for (uint32_t i = tid; i < 256u; i += NT) hist[i] = 0u;
      __syncthreads();
      for (uint32_t j = tid; j < n; j += NT) {
        const uint64_t c = get(j);
        const uint32_t t = uint32_t(c >> 32);
        if (uint32_t(c) == kstar && (t >> (shift + 8)) == (prefix >> (shift + 8)))
          atomicAdd(&hist[(t >> shift) & 0xffu], 1u);
      }
      __syncthreads();
      if (tid < 64) bottom_bin_wave(hist, m, out);
      __syncthreads();
      prefix |= out[0] << shift;
      m -= out[1];
      __syncthreads();
    }
    istar = prefix;
  }
  *kstar_out = kstar;
  *istar_out = istar;
}

// Selection mode of sequence b: kk tokens to select among n_cand candidates.
struct RowMode {
  int Tb, n_cand, kk, nW;
  __device__ bool select() const { return kk > 0 && kk < n_cand; }
};
__device__ __forceinline__ RowMode row_mode(const PipeArgs& a, int b) {
  RowMode m;
  m.n_cand = candidates_of(a.at.seq_lens, b, a.at.t_max, a.window, &m.Tb);
  m.kk = a.topk < m.n_cand ? a.topk : m.n_cand;
  m.nW = a.window < m.Tb ? a.window : m.Tb;
  return m;
}

constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }

// 16 bytes at an 8-byte aligned address (two candidate slots)
typedef uint32_t u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));

// Projection of the group's queries: the G query rows and P[h] (in chunks of
// at most 4096 floats, rows of d in order) are staged in shared memory with all
// loads of a chunk issued at once, then
//   qp[g][i] = sum_d q[b, h*G + g, d] * P[h, d, i]
// with the d-sum split over 256 / (G*R) threads, four running sums per thread
// (d, d+1, d+2, d+3) carried across chunks, added as (s0 + s1) + (s2 + s3), and
// the parts added in order: the arithmetic of the stand-alone score kernel.
// `issued()` runs right after the loads of the first chunk are issued: loads
// the caller issues there complete after the projection's own (memory
// operations complete in order), so the projection never waits for them.
template <int D, int R, int G>
struct QpSmem {
  static constexpr int PCH = D * R <= 4096 ? D * R : 4096;  // floats of P per chunk
  float P[PCH];
  float q[G * D];
  float part[256];
  float qp[G * R];
};

template <int D, int R, int G, typename F>
__device__ __forceinline__ void project_query_staged(const PipeArgs& a, int b, int h, QpSmem<D, R, G>& sm, F issued) {
  constexpr int PCH = QpSmem<D, R, G>::PCH;
  constexpr int DCH = PCH / R;  // rows of d per chunk
  constexpr int NCH = D / DCH;
  constexpr int NP = PCH / 1024;           // 16-byte loads of a chunk per thread
  constexpr int NQ = (G * D + 255) / 256;  // query elements per thread
  constexpr int GR = G * R;
  constexpr int PARTS = 256 / GR;
  constexpr int DPER = D / PARTS;
  static_assert(PCH % 1024 == 0 && GR <= 256 && DPER % 4 == 0 && DCH % 4 == 0, "staging shape");
  const float* Ph = a.P + size_t(h) * D * R;
  const size_t q0 = (size_t(b) * a.at.Hq + size_t(h) * G) * D;
  float qv[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) qv[i] = load_elem(a.at.q, q0 + min(i * 256 + int(threadIdx.x), G * D - 1), a.q_dtype);
  const int o = threadIdx.x % GR, part = threadIdx.x / GR;
  const int g = o / R, i = o - g * R;
  const int d_lo = part * DPER, d_hi = d_lo + DPER;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 1
  for (int c = 0; c < NCH; ++c) {
    uint4 pv[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k)
      pv[k] = load16(reinterpret_cast<const uint4*>(Ph + size_t(c) * PCH) + k * 256 + threadIdx.x);
    if (c == 0) issued();
    if (c > 0) __syncthreads();  // the previous chunk is no longer read
#pragma unroll
    for (int k = 0; k < NP; ++k) reinterpret_cast<uint4*>(sm.P)[k * 256 + threadIdx.x] = pv[k];
    if (c == 0) {
#pragma unroll
      for (int k = 0; k < NQ; ++k)
        if (k * 256 + int(threadIdx.x) < G * D) sm.q[k * 256 + threadIdx.x] = qv[k];
    }
    __syncthreads();
    const float* qg = sm.q + g * D;
    const int lo = max(d_lo, c * DCH), hi = min(d_hi, (c + 1) * DCH);
    for (int d = lo; d < hi; d += 4) {
      const int dl = d - c * DCH;
      a0 = fmaf(qg[d + 0], sm.P[(dl + 0) * R + i], a0);
      a1 = fmaf(qg[d + 1], sm.P[(dl + 1) * R + i], a1);
      a2 = fmaf(qg[d + 2], sm.P[(dl + 2) * R + i], a2);
      a3 = fmaf(qg[d + 3], sm.P[(dl + 3) * R + i], a3);
    }
  }
  sm.part[threadIdx.x] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  for (int j = threadIdx.x; j < GR; j += 256) {
    float acc = 0.f;
    for (int pp = 0; pp < PARTS; ++pp) acc += sm.part[pp * GR + j];
    sm.qp[j] = acc;
  }
  __syncthreads();
}

template <int KPT, int R, int GE, int D, int G, int KVT>
struct Pipe {
  using S = ScanShape<KPT, R>;
  static constexpr int TS = kPipeTileTokens > 2 * S::PER_ITER ? kPipeTileTokens : 2 * S::PER_ITER;  // tokens per tile
  static constexpr int NIT = TS / S::PER_ITER;  // workgroup steps per tile
  static_assert(kPipeMaxItem % TS == 0 && NIT % 2 == 0, "score items are whole tiles of whole step pairs");
  // sample size: two batches of whole steps
  static constexpr int NSAMP = kPipeSampleTokens > 2 * S::PER_ITER ? kPipeSampleTokens : 2 * S::PER_ITER;
  static constexpr int NIT_S = NSAMP / S::PER_ITER;
  static constexpr int RT = kResolveThreads, RW = RT / 64;  // resolve workgroup: threads, waves
  using Qp = QpSmem<D, R, G>;

  struct SampleSmem {
    Qp qp;
    uint32_t keys[NSAMP];
    alignas(16) uint32_t hist[2048];
    uint32_t out[2];
    float apart[256];  // the new key's projection: per-thread partial sums
    uint32_t akp[R];   // and its rounded coordinates
  };
  struct ScoreSmem {
    union {
      Qp qp;
      uint32_t keys[kPipeMaxItem];  // keys of the item's tokens, token order
    };
    uint32_t l_key;
    int claim;
  };
  struct ResolveSmem {
    uint64_t cand[kPipeCandLds + 1];  // (token << 32 | key) of the candidates by ordinal; a dummy slot
    uint32_t tab[kPipeMaxTiles];      // candidate prefix per tile
    alignas(16) uint32_t hist[2048 + 1];  // histograms of the cut; a dummy bin
    alignas(16) uint32_t bin_key[kPipeCutList];  // the candidates of the cut's bin: keys
    alignas(16) uint32_t bin_ord[kPipeCutList];  // and ordinals
    uint32_t wcnt[2][kPipeCandLds / 64];  // flagged candidates per 64 ordinals (two rounds)
    uint32_t wsum[2][kResolveThreads / 64], wmin[kResolveThreads / 64], wmax[kResolveThreads / 64];
    uint32_t scan[kResolveThreads / 64];
    uint32_t out[2];
    uint32_t n_bin;
  };
  static constexpr size_t kSmemScan = cmax(sizeof(SampleSmem), sizeof(ScoreSmem));

  static __device__ const char* kp_row(const PipeArgs& a, int row) {
    return reinterpret_cast<const char*>(a.kp) + size_t(row) * a.at.t_max * R * S::EB;
  }
  static __device__ uint32_t* state(const PipeArgs& a, int row) {
    return a.at.row_state + size_t(row) * kRowStateWords;
  }
  static __device__ uint64_t* l_word(const PipeArgs& a, int row) {
    return reinterpret_cast<uint64_t*>(state(a, row) + PW_L);
  }

  // Rows with nothing to choose: every candidate (kk == n_cand) or none (kk == 0),
  // plus the window (read by the next launch: plain stores).
  static __device__ void resolve_trivial(const PipeArgs& a, int row, const RowMode& md) {
    int32_t* out = a.at.idx + size_t(row) * a.at.idx_stride;
    for (int j = threadIdx.x; j < md.nW; j += 256) out[md.kk + j] = md.Tb - md.nW + j;
    for (int t = threadIdx.x; t < md.kk; t += 256) out[t] = t;
    if (threadIdx.x == 0) const_cast<int32_t*>(a.at.n_sel)[row] = md.kk + md.nW;
  }

  // ---- APPEND (the step's new token, in the sample of its row) ---------------------------
  // The new K and V rows of (b, h) go to the caches at t = pos[b] and the key
  // is projected into the scoring cache with the arithmetic of the stand-alone
  // append (thread (o, part): an fma chain over d in [part*DPER, +DPER), then
  // the parts summed in order, rounded to the cache's type).  The sample does
  // this after it has published the row's threshold (the threshold is on
  // every score run's path, the new row only on one's).  The projected row is
  // stored with device-scope stores and waited for before the row's word is
  // marked (kLwAppended): the score run that holds the token waits for that
  // mark, then re-scores the token's step from the stored row.
  static constexpr int kAppendParts = 256 / R;
  static_assert(D % kAppendParts == 0, "append slices");
  static __device__ __forceinline__ void append_row(const PipeArgs& a, int b, int h, SampleSmem& sm) {
    constexpr int EB = Elem<KVT>::bytes, DPER = D / kAppendParts;
    const int o = threadIdx.x % R, part = threadIdx.x / R;
    const int d0 = part * DPER;
    const char* src = reinterpret_cast<const char*>(a.k_new) + (size_t(b) * a.at.Hkv + h) * D * EB;
    const char* vsrc = reinterpret_cast<const char*>(a.v_new) + (size_t(b) * a.at.Hkv + h) * D * EB;
    const float* Pc = a.P + size_t(h) * D * R + o;
    float kv[DPER], pv[DPER];
#pragma unroll
    for (int i = 0; i < DPER; ++i) {
      if constexpr (KVT == 1) kv[i] = bf16_lo(uint32_t(reinterpret_cast<const uint16_t*>(src)[d0 + i]));
      else kv[i] = reinterpret_cast<const float*>(src)[d0 + i];
      pv[i] = Pc[size_t(d0 + i) * R];
    }
    constexpr int N16 = D * EB / 16;
    uint4 kc16 = make_uint4(0u, 0u, 0u, 0u), vc16 = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x < N16) {
      kc16 = load16(src + size_t(threadIdx.x) * 16);
      vc16 = load16(vsrc + size_t(threadIdx.x) * 16);
    }
    const int t = a.pos[b];
    const bool ok = t >= 0 && t < a.at.t_max;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < DPER; ++i) acc = fmaf(kv[i], pv[i], acc);
    sm.apart[threadIdx.x] = acc;
    if (ok && threadIdx.x < N16) {
      const size_t row_off = ((size_t(b) * a.at.t_max + t) * a.at.Hkv + h) * D * EB + size_t(threadIdx.x) * 16;
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.k_w) + row_off) = kc16;
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.v_w) + row_off) = vc16;
    }
    __syncthreads();
    if (threadIdx.x < R) {
      float sum = 0.f;
      for (int pp = 0; pp < kAppendParts; ++pp) sum += sm.apart[pp * R + threadIdx.x];
      sm.akp[threadIdx.x] = KPT == 1   ? uint32_t(f32_to_bf16_rne(sum))
                            : KPT == 2 ? f32_to_e4m3_sat(sum)
                                       : __float_as_uint(sum);
    }
    __syncthreads();
    if (ok) {
      char* kprow = reinterpret_cast<char*>(a.kp_w) + ((size_t(b) * a.at.Hkv + h) * a.at.t_max + t) * R * S::EB;
      if constexpr (KPT == 1) {
        if (threadIdx.x < R / 2)
          publish(reinterpret_cast<uint32_t*>(kprow) + threadIdx.x,
                  sm.akp[2 * threadIdx.x] | (sm.akp[2 * threadIdx.x + 1] << 16));
      } else if constexpr (KPT == 2) {
        if (threadIdx.x < R / 4) {
          const uint32_t* c = sm.akp + 4 * threadIdx.x;
          publish(reinterpret_cast<uint32_t*>(kprow) + threadIdx.x, c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24));
        }
      } else {
        if (threadIdx.x < R) publish(reinterpret_cast<uint32_t*>(kprow) + threadIdx.x, sm.akp[threadIdx.x]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the projected row is stored before anything this row publishes
    __syncthreads();
  }
  // One scan step's loads through device-scope loads (they see the row the
  // sample appended in this launch).
  static __device__ void load_step_fresh(const char* kr, int base, int t_end, uint4 (&v)[S::U]) {
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int t = min(base + slot_token<KPT, R>(u), t_end - 1);
      const uint64_t* p = reinterpret_cast<const uint64_t*>(kr + size_t(t) * R * S::EB + slot_byte<KPT, R>(u));
      const uint64_t lo = consume(p), hi = consume(p + 1);
      v[u] = make_uint4(uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32));
    }
  }
  // Re-scores the step of [t_begin, t_end) that holds the appended token (if
  // any), with the row as now stored; keys[] holds the range's keys.
  static __device__ __forceinline__ void rescore_new(const PipeArgs& a, int row, int b, const char* kr,
                                                     int t_begin, int t_end, const QFrag<KPT, R, GE>& qf,
                                                     uint32_t* keys, uint64_t deadline) {
    if (!a.k_new) return;
    const int t = a.pos[b];
    if (t < t_begin || t >= t_end) return;
    if (threadIdx.x == 0) {  // the sample has stored the row
      uint64_t lw = consume(l_word(a, row));
      while (!(lw & kLwAppended) && !past(deadline)) {
        __builtin_amdgcn_s_sleep(1);
        lw = consume(l_word(a, row));
      }
      if (!(lw & kLwAppended)) flag_error(a);
    }
    __syncthreads();
    const int st = (t - t_begin) / S::PER_ITER;
    uint4 v[S::U];
    load_step_fresh(kr, t_begin + st * S::PER_ITER, t_end, v);
    uint32_t* kst = keys + st * S::PER_ITER;
    score_loads<KPT, R, GE>(v, qf, G, [&](int toff, float sc) { kst[toff] = score_key(sc); });
  }

  // ---- SAMPLE -----------------------------------------------------------------------------
  // The rank m of the row's threshold among NSAMP evenly strided tokens (the
  // threshold is their m-th largest key: k's expected share of the sample
  // plus four standard deviations and a margin), or 0 when every token is a
  // candidate (a short row, or a budget the sample cannot usefully bound).
  static __device__ __forceinline__ int sample_rank(const RowMode& md) {
    if (md.n_cand <= kPipeSampleMin) return 0;
    const double E = double(NSAMP) * md.kk / md.n_cand;  // expected sample tokens above the k-th score
    const int m = int(ceil(E + 4.0 * sqrt(E) + 8.0));
    return m < NSAMP ? m : 0;
  }
  static __device__ __forceinline__ void sample(const PipeArgs& a, int row, SampleSmem& sm) {
    const int b = row / a.at.Hkv, h = row - b * a.at.Hkv;
    const RowMode md = row_mode(a, b);
    if (!md.select()) {
      resolve_trivial(a, row, md);
      if (a.k_new) append_row(a, b, h, sm);  // no score run reads this row
      return;
    }
    uint32_t L = 0;  // every token is a candidate unless a sample allows a higher threshold
    const int m = sample_rank(md);
    if (m > 0) {
      const int n_samp = NSAMP;  // n_cand > NSAMP here
      const int stride = md.n_cand / n_samp;
      {
        // the sampled projected keys are requested before the query projection
        const char* kr = kp_row(a, row);
        constexpr int HALF = NIT_S / 2;  // steps per batch of loads
        auto load_half = [&](int it0, uint4 (&v)[HALF][S::U]) {
#pragma unroll
          for (int it = 0; it < HALF; ++it)
#pragma unroll
            for (int u = 0; u < S::U; ++u) {
              const int i = (it0 + it) * S::PER_ITER + slot_token<KPT, R>(u);
              v[it][u] = load16_nt(kr + size_t(i) * stride * R * S::EB + slot_byte<KPT, R>(u));
            }
        };
        uint4 v[HALF][S::U];
        project_query_staged<D, R, G>(a, b, h, sm.qp, [&] { load_half(0, v); });
        // left for the select/attend launch, in case the row has to be re-selected exactly
        for (int j = threadIdx.x; j < G * R; j += 256) a.qp_pub[size_t(row) * G * R + j] = sm.qp.qp[j];
        QFrag<KPT, R, GE> qf;
        load_qfrag<KPT, R, GE>([&](int i) { return sm.qp.qp[i]; }, G, qf);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint4 w[HALF][S::U];
          if (half == 0) load_half(HALF, w);
#pragma unroll
          for (int it = 0; it < HALF; ++it) {
            const int i0 = (half * HALF + it) * S::PER_ITER;
            score_loads<KPT, R, GE>(v[it], qf, G, [&](int toff, float sc) { sm.keys[i0 + toff] = score_key(sc); });
          }
          if (half == 0) {
#pragma unroll
            for (int it = 0; it < HALF; ++it)
#pragma unroll
              for (int u = 0; u < S::U; ++u) v[it][u] = w[it][u];
          }
        }
        __syncthreads();
        uint32_t kstar, istar;
        kth_cut<256>([&](uint32_t j) { return uint64_t(sm.keys[j]); }, uint32_t(n_samp), uint32_t(m), false,
                     sm.hist, sm.out, &kstar, &istar);
        L = kstar;
      }
    }
    if (threadIdx.x == 0) publish(l_word(a, row), kLwSet | L);
    if (a.k_new) {
      append_row(a, b, h, sm);
      if (threadIdx.x == 0) publish(l_word(a, row), kLwSet | kLwAppended | L);
    }
  }

  // ---- SCORE ------------------------------------------------------------------------------
  // Scores tokens [t_begin, t_end) of the row into keys[t - t_begin] (token
  // order).  pre[j] holds the loads of step j, already issued: kPipePF steps
  // stay in flight, step st + kPipePF being requested as soon as step st is
  // scored.  Loads carry no per-lane branch (tokens past the end re-read the
  // last one).
  // `late()` runs once, before the last whole group of steps (or before the
  // remaining steps when there is no whole group): a load it issues is in
  // flight behind the range's last key loads.
  template <typename Late>
  static __device__ void scan_keys(const char* kr, int t_begin, int t_end, const QFrag<KPT, R, GE>& qf,
                                   uint4 (&pre)[kPipePF][S::U], uint32_t* keys, Late late) {
    const int n_steps = (t_end - t_begin + S::PER_ITER - 1) / S::PER_ITER;
    // whole groups of kPipePF steps with every reload unconditional (past the
    // end they re-read the last token), so the wait before each step's use
    // counts the same loads on every path; then the remaining steps
    int st0 = 0;
    if (n_steps < kPipePF) late();
    for (; st0 + kPipePF <= n_steps; st0 += kPipePF) {
      if (st0 + 2 * kPipePF > n_steps) late();
#pragma unroll
      for (int j = 0; j < kPipePF; ++j) {
        uint32_t* kst = keys + (st0 + j) * S::PER_ITER;
        score_loads<KPT, R, GE>(pre[j], qf, G, [&](int toff, float sc) { kst[toff] = score_key(sc); });
        load_step(kr, t_begin + (st0 + j + kPipePF) * S::PER_ITER, t_end, pre[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kPipePF; ++j) {
      if (st0 + j < n_steps) {
        uint32_t* kst = keys + (st0 + j) * S::PER_ITER;
        score_loads<KPT, R, GE>(pre[j], qf, G, [&](int toff, float sc) { kst[toff] = score_key(sc); });
      }
    }
  }
  // the first kPipePF steps of [t_begin, t_end)
  static __device__ __forceinline__ void load_first(const char* kr, int t_begin, int t_end,
                                                    uint4 (&pre)[kPipePF][S::U]) {
#pragma unroll
    for (int j = 0; j < kPipePF; ++j) load_step(kr, t_begin + j * S::PER_ITER, t_end, pre[j]);
  }
  static __device__ void load_step(const char* kr, int base, int t_end, uint4 (&v)[S::U]) {
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int t = min(base + slot_token<KPT, R>(u), t_end - 1);
      v[u] = load16_nt(kr + size_t(t) * R * S::EB + slot_byte<KPT, R>(u));
    }
  }

  // Writes the tokens of [t_begin, t_end) (whole tiles from t_begin) whose key
  // in keys[] is >= thr to their tiles' candidate slots, in token order, and
  // the tile counts (plain stores: read after the launch boundary, or by the
  // workgroup that wrote them).  Each wave compacts whole tiles in rounds of 64
  // tokens (lane l takes token 64 k + l of round k, so the key reads are
  // conflict-free); a ballot per round gives the positions.  A tile's keys
  // are all read into registers before its first round: each round's store
  // sits behind a branch, and a shared-memory read issued after one would
  // wait out its full latency in every round.
  template <int NW = 4>
  static __device__ void emit_keys(const PipeArgs& a, int row, int t_begin, int t_end, uint32_t thr,
                                   const uint32_t* keys) {
    constexpr int PL = TS / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_sub = (t_end - t_begin + TS - 1) / TS;
    const int tile0 = t_begin / TS;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int s = wave; s < n_sub; s += NW) {
      const int t0 = t_begin + s * TS;
      const int n_tok = min(TS, t_end - t0);
      const uint32_t* kk = keys + s * TS;
      uint64_t* slot = a.cand + size_t(row) * a.at.t_max + size_t(tile0 + s) * TS;
      uint32_t kv[PL];
#pragma unroll
      for (int k = 0; k < PL; ++k) kv[k] = kk[k * 64 + lane];
      uint32_t pos = 0;
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const int i = k * 64 + lane;
        const uint32_t key = kv[k];
        const bool take = i < n_tok && key >= thr;
        const unsigned long long m = __ballot(take);
        if (take) slot[pos + uint32_t(__popcll(m & below))] = (uint64_t(uint32_t(t0 + i)) << 32) | key;
        pos += uint32_t(__popcll(m));
      }
      if (lane == 0) a.tile_cnt[size_t(row) * a.n_tiles + tile0 + s] = pos;
    }
  }

  // Scores tokens [t_begin, t_end) of the row (t_begin on a tile boundary,
  // t_end <= n_cand) with one query projection, in items of at most
  // kPipeMaxItem tokens (the key buffer), and emits each item's candidates.
  // The row's threshold is waited for after the first item's scan.
  static __device__ void score_range(const PipeArgs& a, int row, int t_begin, int t_end, char* smem,
                                     uint64_t deadline, bool split_tail) {
    const int b = row / a.at.Hkv, h = row - b * a.at.Hkv;
    ScoreSmem& sm = *reinterpret_cast<ScoreSmem*>(smem);
    const char* kr = kp_row(a, row);
    uint4 pre[kPipePF][S::U];
    uint64_t lw = 0;
    // With split_tail, a range of four tiles or more keeps its last two
    // tiles for an item of their own: the items before emit their candidates
    // while the next item's first keys are in flight, so only two tiles'
    // emission follows the range's last key loads.  (The segments of the
    // range split, already cut at row boundaries, keep whole items: each
    // extra item boundary drains the load pipeline once.  So do FP8 keys,
    // whose scan is bound by instruction issue rather than by the tail.)
    const int n_t = (t_end - t_begin + TS - 1) / TS;
    const int tail0 = split_tail && !S::F8 && n_t >= 4 ? t_begin + (n_t - 2) * TS : t_end;
    auto item_end = [&](int x) { return x < tail0 ? min(x + kPipeMaxItem, tail0) : t_end; };
    int tb = t_begin, te = item_end(t_begin);
    project_query_staged<D, R, G>(a, b, h, sm.qp, [&] {
      load_first(kr, tb, te, pre);  // in flight during the query projection
      if (threadIdx.x == 0) lw = consume(l_word(a, row));
    });
    QFrag<KPT, R, GE> qf;
    load_qfrag<KPT, R, GE>([&](int i) { return sm.qp.qp[i]; }, G, qf);
    __syncthreads();  // the projection's shared memory becomes the key buffer
    for (;;) {
      // the row's threshold is read again behind the first item's last key
      // loads, so it is usually in hand when the item's keys are
      scan_keys(kr, tb, te, qf, pre, sm.keys, [&] {
        if (tb == t_begin && threadIdx.x == 0 && (lw >> 32) == 0) lw = consume(l_word(a, row));
      });
      if (tb == t_begin) {  // the row's threshold (its sample was handed out before any score work)
        if (threadIdx.x == 0) {
          while ((lw >> 32) == 0 && !past(deadline)) {
            __builtin_amdgcn_s_sleep(1);
            lw = consume(l_word(a, row));
          }
          if ((lw >> 32) == 0) flag_error(a);
          sm.l_key = uint32_t(lw);
        }
        __syncthreads();
      }
      rescore_new(a, row, b, kr, tb, te, qf, sm.keys, deadline);
      __syncthreads();
      const int nb = te, ne = te < t_end ? item_end(te) : t_end;
      if (nb < t_end) load_first(kr, nb, ne, pre);  // in flight during the emission
      emit_keys(a, row, tb, te, sm.l_key, sm.keys);
      if (nb >= t_end) return;
      tb = nb;
      te = ne;
      __syncthreads();  // every wave is done with keys[]
    }
  }

  // ---- SPLIT OF THE SCORE WORK -----------------------------------------------------------
  // The rows' candidate tiles go to the score workgroups in proportion to the
  // rows' lengths: sequence b's Hkv rows of tiles_of(b) tiles each get
  // w(b) = floor(spare * tiles_of(b) / N) + 1 workgroups per row (N: the
  // tiles of all rows; spare: the score workgroups beyond one per row), and
  // workgroup j of a row scans its tiles [j T / w, (j + 1) T / w): one row and
  // one query projection per workgroup, and about N / spare tiles each,
  // whatever the mix of lengths.  With fewer score workgroups than rows, the
  // rows' tiles are instead laid end to end (sequence b, then KV head, then
  // tile) and split into equal contiguous ranges.
  static __device__ __forceinline__ int tiles_of(const PipeArgs& a, int b) {
    const RowMode md = row_mode(a, b);
    return md.select() ? (md.n_cand + TS - 1) / TS : 0;
  }
  struct FlatSmem {
    uint32_t wsum[256 / 64];
    uint32_t found[2];
  };
  // Sum over sequences of cnt(b) (every thread gets it).
  template <typename Cnt>
  static __device__ __forceinline__ uint32_t seq_total(const PipeArgs& a, FlatSmem& fs, Cnt cnt) {
    const int B = a.n_rows / a.at.Hkv;
    uint32_t mine = 0;
    for (int b = threadIdx.x; b < B; b += 256) mine += cnt(b);
    uint32_t total;
    block_exclusive_scan<4>(mine, fs.wsum, &total);
    return total;
  }
  // The sequence b whose run of the sums of cnt holds g, and g's offset in it
  // (g below the total).
  template <typename Cnt>
  static __device__ __forceinline__ void seq_locate(const PipeArgs& a, FlatSmem& fs, uint32_t g, Cnt cnt, int* b_out,
                                                    uint32_t* o_out) {
    const int B = a.n_rows / a.at.Hkv;
    uint32_t base = 0;
    for (int b0 = 0; b0 < B; b0 += 256) {
      const int b = b0 + int(threadIdx.x);
      const uint32_t c = b < B ? cnt(b) : 0u;
      uint32_t chunk;
      const uint32_t ex = base + block_exclusive_scan<4>(c, fs.wsum, &chunk);
      if (c && g >= ex && g < ex + c) {  // one thread
        fs.found[0] = uint32_t(b);
        fs.found[1] = g - ex;
      }
      base += chunk;
      __syncthreads();
      if (g < base) break;  // uniform
    }
    __syncthreads();
    *b_out = int(fs.found[0]);
    *o_out = fs.found[1];
    __syncthreads();  // found[] is reused
  }
  static __device__ void score_split(const PipeArgs& a, char* smem, FlatSmem& fs, uint64_t deadline) {
    const int grid = int(gridDim.x);
    // workgroups that sample sit out the split when the others are many enough
    const int first = a.samples_in_scan && grid >= 2 * a.n_rows ? a.n_rows : 0;
    const int s = int(blockIdx.x) - first;
    if (s < 0) return;
    const uint32_t W = uint32_t(grid - first);
    const uint32_t Hkv = uint32_t(a.at.Hkv);
    // Every sequence with the same tile count (the usual batch): the split in
    // closed form, without the scans.  Runs of `it` tiles, ceil(nt / it) of
    // them per row; run j of row r is score workgroup j n_rows + (r - j mod
    // n_rows), so every row's first runs are dispatched first and a row's
    // runs rotate over the XCDs.
    {
      const int B = a.n_rows / a.at.Hkv, lane = int(threadIdx.x & 63);
      const int nt0 = tiles_of(a, 0);
      bool same = true;  // a wave vote: every wave reads every length, no barrier
      int lane_cand = 0;  // candidates of sequence `lane` (B <= 64)
      for (int b = lane; b < B; b += 64) {
        const RowMode mb = row_mode(a, b);
        same = same && (mb.select() ? (mb.n_cand + TS - 1) / TS : 0) == nt0;
        if (b == lane) lane_cand = mb.n_cand;
      }
      if (__all(same)) {
        if (nt0 == 0) return;
        const int per_row = int(W) / a.n_rows;
        if (per_row >= 1) {
          const int it = (nt0 + per_row - 1) / per_row, runs = (nt0 + it - 1) / it;
          if (s >= a.n_rows * runs) return;
          const int j = s / a.n_rows, r = (s - j * a.n_rows + j) % a.n_rows;
          const int bq = r / a.at.Hkv;
          const int n_cand = B <= 64 ? __shfl(lane_cand, bq) : row_mode(a, bq).n_cand;
          score_range(a, r, j * it * TS, min(min(j * it + it, nt0) * TS, n_cand), smem, deadline, true);
          return;
        }
      }
    }
    const uint32_t N = seq_total(a, fs, [&](int b) { return Hkv * uint32_t(tiles_of(a, b)); });
    const uint32_t rows_live = seq_total(a, fs, [&](int b) { return tiles_of(a, b) ? Hkv : 0u; });
    if (N == 0) return;
    const uint64_t spare = W >= rows_live ? W - rows_live : 0u;
    auto per_row = [&](int b) -> uint32_t {
      const uint32_t t = uint32_t(tiles_of(a, b));
      return t ? uint32_t(spare * t / N) + 1u : 0u;
    };
    // Whole workgroups per row round each row's share: a long row's runs can
    // end up several tiles longer than the even share ceil(N / W) (16 against
    // 14 tiles in a batch of 8K..128K rows), and the scan lasts as long as its
    // longest run.  Then the equal contiguous ranges below serve better, at
    // the cost of a second query projection in the workgroups whose range
    // crosses a row boundary.
    const uint32_t even = (N + W - 1) / W;
    const bool uneven =
        W >= rows_live && seq_total(a, fs, [&](int b) {
          const uint32_t t = uint32_t(tiles_of(a, b)), w = per_row(b);
          return t && (t + w - 1) / w > even + 1u ? 1u : 0u;
        }) != 0u;
    if (W >= rows_live && !uneven) {
      if (uint32_t(s) >= seq_total(a, fs, [&](int b) { return Hkv * per_row(b); })) return;
      int b;
      uint32_t o;
      seq_locate(a, fs, uint32_t(s), [&](int b) { return Hkv * per_row(b); }, &b, &o);
      const uint32_t w = per_row(b), h = o / w, j = o - h * w;
      const RowMode md = row_mode(a, b);
      const uint32_t nt = uint32_t(tiles_of(a, b));
      const int t0 = int(uint64_t(nt) * j / w), t1 = int(uint64_t(nt) * (j + 1) / w);
      if (t1 > t0) score_range(a, b * a.at.Hkv + int(h), t0 * TS, min(t1 * TS, md.n_cand), smem, deadline, true);
      return;
    }
    // fewer score workgroups than rows, or an uneven per-row split: equal
    // contiguous ranges of the rows' tiles laid end to end
    if (s == 0 && threadIdx.x == 0) __hip_atomic_fetch_add(a.at.queue + QW_RANGE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t g = uint32_t(uint64_t(N) * uint32_t(s) / W);
    const uint32_t g1 = uint32_t(uint64_t(N) * uint32_t(s + 1) / W);
    if (g >= g1) return;
    int b;
    uint32_t o;
    seq_locate(a, fs, g, [&](int b) { return Hkv * uint32_t(tiles_of(a, b)); }, &b, &o);
    while (g < g1) {  // one row segment at a time (sequences with nothing to score hold no tiles)
      const RowMode md = row_mode(a, b);
      const uint32_t nt = uint32_t(tiles_of(a, b));
      if (nt == 0 || o >= Hkv * nt) {
        ++b;
        o = 0;
        continue;
      }
      const uint32_t h = o / nt, t0 = o - h * nt;
      const uint32_t seg = min(nt - t0, g1 - g);
      score_range(a, b * a.at.Hkv + int(h), int(t0) * TS, min(int(t0 + seg) * TS, md.n_cand), smem, deadline,
                  false);
      __syncthreads();
      g += seg;
      o += seg;
    }
  }

  // ---- SELECTION (second launch) ----------------------------------------------------------
  // Gathers the row's candidates into shared memory by ordinal (token order).
  // Each wave takes kPipeGatherTiles tiles a round and issues every load of the
  // round at once: the tiles' counts (one per lane) and their first 64 SL slots
  // (SL 8-byte loads per lane and tile: a tile's candidates are contiguous
  // from the start of its slot; about 40 at 128K context and k = 2048, about
  // 100 at k = 8192 or at 32K context, where SL = 2; slots past the count are
  // read but not used, and the candidate buffer has kCandPad slots past its
  // last row, so no load needs a bound; a tile with more takes further round
  // trips).  A shuffle scan of the counts and the wave totals give the tiles'
  // first ordinals, kept in sm.tab.  Stores of unused lanes go to a dummy
  // slot.  Returns the number of candidates C; *kmin / *kmax: their smallest /
  // largest key (C > 0).  FRESH: the slots and counts were rewritten by this
  // workgroup after an earlier gather, so they are read with device-scope
  // loads.
  static_assert(kCandPad >= 128, "the gather reads up to 128 slots from a tile's start");
  static __device__ __forceinline__ void minmax_block(ResolveSmem& sm, uint32_t lo, uint32_t hi, uint32_t* kmin,
                                                      uint32_t* kmax) {
    const int wave = threadIdx.x >> 6;
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    sm.wmin[wave] = lo;
    sm.wmax[wave] = hi;
    __syncthreads();  // also: every gathered candidate is in shared memory
    lo = 0xffffffffu;
    hi = 0u;
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      lo = min(lo, sm.wmin[w]);
      hi = max(hi, sm.wmax[w]);
    }
    *kmin = lo;
    *kmax = hi;
  }
  template <bool FRESH, int SL>
  static __device__ __forceinline__ uint32_t gather(const PipeArgs& a, int row, int n_tiles_row, ResolveSmem& sm,
                                                    uint32_t* kmin, uint32_t* kmax) {
    constexpr int UB = kPipeGatherTiles;
    const uint32_t lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t* cnt_row = a.tile_cnt + size_t(row) * a.n_tiles;
    const uint64_t* slots = a.cand + size_t(row) * a.at.t_max;
    uint32_t run = 0, lo = 0xffffffffu, hi = 0u;
    auto put = [&](bool ok, uint32_t pos, uint64_t c) {
      const uint32_t key = uint32_t(c);
      lo = min(lo, ok ? key : 0xffffffffu);
      hi = max(hi, ok ? key : 0u);
      sm.cand[(ok && pos < uint32_t(kPipeCandLds)) ? pos : uint32_t(kPipeCandLds)] = c;
    };
    int parity = 0;
    for (int r0 = 0; r0 < n_tiles_row; r0 += RW * UB, parity ^= 1) {
      const int t0 = r0 + wave * UB;
      const int tl = min(t0 + int(lane & (UB - 1)), n_tiles_row - 1);
      const bool own = lane < uint32_t(UB) && t0 + int(lane) < n_tiles_row;
      uint32_t my_cnt = FRESH ? consume(cnt_row + tl) : cnt_row[tl];
      my_cnt = own ? my_cnt : 0u;
      uint64_t v0[UB][SL];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int t = min(t0 + u, n_tiles_row - 1);  // past the row's tiles: count 0
#pragma unroll
        for (int q = 0; q < SL; ++q) {
          const uint64_t* src = slots + size_t(t) * TS + q * 64 + lane;
          v0[u][q] = FRESH ? consume(src) : *src;
        }
      }
      const uint32_t incl = wave_scan_incl(my_cnt);  // over the lanes that own tiles
      sm.wsum[parity][wave] = uint32_t(__builtin_amdgcn_readlane(int(incl), UB - 1));
      __syncthreads();
      uint32_t wbase = run, rtot = 0;
#pragma unroll
      for (int w = 0; w < RW; ++w) {
        const uint32_t c = sm.wsum[parity][w];
        wbase += (w < wave) ? c : 0u;
        rtot += c;
      }
      const uint32_t excl = incl - my_cnt;
      if (own) sm.tab[t0 + lane] = wbase + excl;
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const uint32_t cnt_u = uint32_t(__builtin_amdgcn_readlane(int(my_cnt), u));
        const uint32_t base_u = wbase + uint32_t(__builtin_amdgcn_readlane(int(excl), u));
#pragma unroll
        for (int q = 0; q < SL; ++q) put(q * 64 + lane < cnt_u, base_u + q * 64 + lane, v0[u][q]);
        if (cnt_u > 64u * SL) {  // a crowded tile: the rest of its slot
          const uint64_t* src = slots + size_t(t0 + u) * TS;
          for (uint32_t i = lane + 64u * SL; i < cnt_u; i += 64u) put(true, base_u + i, FRESH ? consume(src + i) : src[i]);
        }
      }
      run += rtot;
    }
    minmax_block(sm, lo, hi, kmin, kmax);
    return run;
  }
  // A row whose every token is a candidate (no sampled threshold): each tile
  // holds all of its tokens, so the row's slots are one contiguous run of
  // n_cand candidates in token order, copied with coalesced loads.  Only the
  // first kPipeCandLds go to shared memory (more are cut in place, through
  // sm.tab, which holds the tiles' first ordinals here too).
  static __device__ __forceinline__ uint32_t gather_all(const PipeArgs& a, int row, int n_cand, int n_tiles_row,
                                                        ResolveSmem& sm, uint32_t* kmin, uint32_t* kmax) {
    constexpr int B = 8;
    const uint64_t* slots = a.cand + size_t(row) * a.at.t_max;
    for (int t = threadIdx.x; t < n_tiles_row; t += RT) sm.tab[t] = uint32_t(t) * TS;
    uint32_t lo = 0xffffffffu, hi = 0u;
    for (int o0 = 0; o0 < n_cand; o0 += B * RT) {
      uint64_t v[B];
#pragma unroll
      for (int u = 0; u < B; ++u) v[u] = slots[min(o0 + u * RT + int(threadIdx.x), n_cand - 1)];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int o = o0 + u * RT + int(threadIdx.x);
        const bool ok = o < n_cand;
        const uint32_t key = uint32_t(v[u]);
        lo = min(lo, ok ? key : 0xffffffffu);
        hi = max(hi, ok ? key : 0u);
        if (ok && o < kPipeCandLds) sm.cand[o] = v[u];
      }
    }
    minmax_block(sm, lo, hi, kmin, kmax);
    return uint32_t(n_cand);
  }

  // The sampled threshold let fewer than kk tokens through: rebuild the row's
  // candidate slots exactly (every key in or above the k-th key's top 11-bit
  // bin), scanning the row twice: once for the histogram of that digit, once
  // to write the candidates.  The scores are the scan's: the group's projected
  // queries left by the sample, the same per-wave arithmetic, with the
  // workgroup's four-wave groups taking the steps of an item in turn.
  static __device__ __forceinline__ void exact_candidates(const PipeArgs& a, int row, const RowMode& md, char* smem,
                                                          bool leader) {
    constexpr int NT = RT, NWG = RT / 256;
    const uint32_t tid = threadIdx.x;
    ScoreSmem& ss = *reinterpret_cast<ScoreSmem*>(smem);
    ResolveSmem& rs = *reinterpret_cast<ResolveSmem*>(smem);
    const float* qp = a.qp_pub + size_t(row) * G * R;
    QFrag<KPT, R, GE> qf;
    load_qfrag<KPT, R, GE>([&](int i) { return qp[i]; }, G, qf);
    for (uint32_t i = tid; i < 2048u; i += NT) rs.hist[i] = 0u;
    __syncthreads();
    const char* kr = kp_row(a, row);
    const int group = int(tid) >> 8;
    for (int pass = 0; pass < 2; ++pass) {
      uint32_t thr = 0;
      if (pass == 1) {
        if (tid < 64) top_bin_wave(rs.hist, uint32_t(md.kk), rs.out);
        __syncthreads();
        thr = rs.out[0] << 21;
        __syncthreads();
      }
      for (int t_begin = 0; t_begin < md.n_cand; t_begin += kPipeMaxItem) {
        const int t_end = min(t_begin + kPipeMaxItem, md.n_cand);
        const int n_steps = (t_end - t_begin + S::PER_ITER - 1) / S::PER_ITER;
        for (int st = group; st < n_steps; st += NWG) {
          uint4 v[S::U];
          load_step(kr, t_begin + st * S::PER_ITER, t_end, v);
          uint32_t* kst = ss.keys + st * S::PER_ITER;
          score_loads<KPT, R, GE>(v, qf, G, [&](int toff, float sc) { kst[toff] = score_key(sc); });
        }
        __syncthreads();
        if (pass == 0) {
          for (int i = int(tid); i < t_end - t_begin; i += NT) atomicAdd(&rs.hist[ss.keys[i] >> 21], 1u);
        } else {
          emit_keys<NT / 64>(a, row, t_begin, t_end, thr, ss.keys);
        }
        __syncthreads();
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (leader && tid == 0) __hip_atomic_fetch_add(a.at.queue + QW_REDO, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Candidate ordinals in shared memory are spread over the RT threads in
  // rounds: ordinal RT i + threadIdx.x belongs to round i, so every pass reads
  // them contiguously.  word_offsets() gives, for a per-ordinal flag, the
  // number of flagged ordinals before each wave's 64 ordinals of each round
  // (one barrier; `buf` alternates between calls): the counts of the RW nper
  // words of 64 ordinals, a scan of them in every wave, then a readlane per
  // round.
  template <int MAXPER, typename Flag>
  static __device__ __forceinline__ void word_offsets(ResolveSmem& sm, int nper, int buf, Flag flag, uint32_t (&off)[MAXPER]) {
    const uint32_t lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      if (i >= nper) { JSSA_ROUNDS_END; }
      sm.wcnt[buf][RW * i + wave] = uint32_t(__popcll(__ballot(flag(i))));  // every lane: the same word
    }
    __syncthreads();
    // lane l holds words WPL l .. WPL l + WPL - 1; word RW i + wave sits at
    // place wave mod WPL of its lane for every round i
    constexpr int WPL = (RW * MAXPER + 63) / 64;
    static_assert(RW % WPL == 0 && WPL * 64 >= RW * MAXPER && RW * MAXPER <= kPipeCandLds / 64, "flag words per lane");
    const int nw = RW * nper;  // <= RW * MAXPER
    uint32_t c[WPL], sum = 0u;
#pragma unroll
    for (int k = 0; k < WPL; ++k) {
      c[k] = int(WPL * lane + k) < nw ? sm.wcnt[buf][WPL * lane + k] : 0u;
      sum += c[k];
    }
    uint32_t ex = wave_scan_incl(sum) - sum;
    const int kw = wave % WPL;
#pragma unroll
    for (int k = 0; k < WPL; ++k) ex += k < kw ? c[k] : 0u;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      if (i >= nper) { JSSA_ROUNDS_END; }
      off[i] = uint32_t(__builtin_amdgcn_readlane(int(ex), (RW * i + wave) / WPL));
    }
  }

  // The cut (K*, I*) when the k-th key's bin of the first digit is too crowded
  // to rank directly: radix passes of 11 bits over d = key - kmin from the top
  // set bit of kmax - kmin down give K*; the `need` lowest ordinals among the
  // keys equal to K* give I*.
  template <int MAXPER>
  static __device__ __forceinline__ void cut_by_passes(ResolveSmem& sm, const uint32_t (&kv)[MAXPER], int nper, uint32_t C,
                                       uint32_t kmin, uint32_t kmax, uint32_t need, uint32_t* kstar_out,
                                       uint32_t* istar_out) {
    const uint32_t tid = threadIdx.x;
    const int nbits = kmax > kmin ? 32 - __clz(kmax - kmin) : 1;
    uint32_t prefix = 0;  // the digits of d* found so far
    for (int hi = nbits; hi > 0; hi -= 11) {
      const int sh = hi > 11 ? hi - 11 : 0;
      for (int i = threadIdx.x; i < 2048; i += RT) sm.hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MAXPER; ++i) {
        if (i >= nper) { JSSA_ROUNDS_END; }
        const uint32_t dv = kv[i] - kmin;
        const bool in = uint32_t(i) * RT + tid < C && (hi >= 32 || (dv >> hi) == (prefix >> hi));
        atomicAdd(&sm.hist[in ? (dv >> sh) & 0x7ffu : 2048u], 1u);
      }
      __syncthreads();
      if (tid < 64) top_bin_wave(sm.hist, need, sm.out);
      __syncthreads();
      prefix |= sm.out[0] << sh;
      need -= sm.out[1];
      __syncthreads();
    }
    const uint32_t kstar = prefix + kmin;
    auto eq = [&](int i) { return uint32_t(i) * RT + tid < C && kv[i] == kstar; };
    uint32_t off[MAXPER];
    word_offsets<MAXPER>(sm, nper, 0, eq, off);
    const uint64_t below = (1ull << (tid & 63)) - 1ull;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      if (i >= nper) { JSSA_ROUNDS_END; }
      const bool e = eq(i);
      const uint64_t mk = __ballot(e);
      if (e && off[i] + uint32_t(__popcll(mk & below)) == need - 1u) sm.out[1] = uint32_t(i) * RT + tid;
    }
    __syncthreads();
    *kstar_out = kstar;
    *istar_out = sm.out[1];
  }

  // The exact cut among C <= MAXPER * RT candidates held in shared memory,
  // then the emission of the selected ones.  Ordinal RT i + threadIdx.x in
  // round i; its key stays in kv[i].  Candidates are in token order, so
  // ranking equal keys by ordinal ranks them by token index.  (Instantiated
  // for half and all of kPipeCandLds: the common budgets keep the smaller
  // register and code footprint.)
  template <int MAXPER, typename Emit>
  static __device__ __forceinline__ void cut_in_lds(ResolveSmem& sm, uint32_t C, uint32_t need, uint32_t kmin,
                                                    uint32_t kmax, Emit emit) {
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const int nper = int((C + RT - 1) / RT);
    uint32_t kv[MAXPER];
    uint32_t kstar, istar;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const uint32_t o = uint32_t(i) * RT + tid;
      kv[i] = i < nper ? uint32_t(sm.cand[min(o, uint32_t(kPipeCandLds))]) : 0u;
    }
    auto live = [&](int i) { return uint32_t(i) * RT + tid < C; };
    // One digit: the top 11 bits of d = key - kmin (the candidates sit in a
    // narrow band at the top, so digits of the key itself would pile them
    // into a few bins).  Everything above the k-th key's bin is taken; the
    // bin's own candidates are ranked directly, by key and then ordinal.
    const int nbits = kmax > kmin ? 32 - __clz(kmax - kmin) : 1;
    const int sh = nbits > 11 ? nbits - 11 : 0;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      if (i >= nper) { JSSA_ROUNDS_END; }
      atomicAdd(&sm.hist[live(i) ? (kv[i] - kmin) >> sh : 2048u], 1u);  // dead lanes: the dummy bin
    }
    __syncthreads();
    if (tid < 64) top_bin_wave(sm.hist, need, sm.out);
    __syncthreads();
    const uint32_t bin = sm.out[0];
    const uint32_t need_bin = need - sm.out[1];  // 1 <= need_bin <= the bin's count
    // the bin's candidates, listed a wave at a time
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      if (i >= nper) { JSSA_ROUNDS_END; }
      const bool inb = live(i) && ((kv[i] - kmin) >> sh) == bin;
      const uint64_t mk = __ballot(inb);
      if (mk) {
        uint32_t b0 = 0;
        if (lane == 0) b0 = atomicAdd(&sm.n_bin, uint32_t(__popcll(mk)));
        b0 = uint32_t(__builtin_amdgcn_readfirstlane(int(b0))) + uint32_t(__popcll(mk & below));
        if (inb && b0 < uint32_t(kPipeCutList)) {
          sm.bin_key[b0] = kv[i];
          sm.bin_ord[b0] = uint32_t(i) * RT + tid;
        }
      }
    }
    __syncthreads();
    const uint32_t m = uint32_t(__builtin_amdgcn_readfirstlane(int(sm.n_bin)));
    if (m <= 64u) {
      // one wave: lane j holds the bin's j-th candidate and counts those
      // ranked above it, four at a time (shared-memory broadcasts)
      if (tid < 64) {
        const uint32_t k = lane < m ? sm.bin_key[lane] : 0u;
        const uint32_t o = lane < m ? sm.bin_ord[lane] : 0xffffffffu;
        uint32_t rank = 0;
        for (uint32_t j = 0; j < m; j += 4) {
          const uint4 k4 = *reinterpret_cast<const uint4*>(&sm.bin_key[j]);
          const uint4 o4 = *reinterpret_cast<const uint4*>(&sm.bin_ord[j]);
          auto above = [&](uint32_t q, uint32_t kj, uint32_t oj) {
            return (j + q < m && (kj > k || (kj == k && oj < o))) ? 1u : 0u;
          };
          rank += above(0, k4.x, o4.x) + above(1, k4.y, o4.y) + above(2, k4.z, o4.z) + above(3, k4.w, o4.w);
        }
        if (lane < m && rank == need_bin - 1u) {
          sm.out[0] = k;
          sm.out[1] = o;
        }
      }
      __syncthreads();
      kstar = sm.out[0];
      istar = sm.out[1];
    } else if (m <= uint32_t(kPipeCutList)) {
      if (tid < m) {
        const uint32_t k = sm.bin_key[tid], o = sm.bin_ord[tid];
        uint32_t rank = 0;
        for (uint32_t j = 0; j < m; ++j) {
          const uint32_t kj = sm.bin_key[j], oj = sm.bin_ord[j];
          rank += (kj > k || (kj == k && oj < o)) ? 1u : 0u;
        }
        if (rank == need_bin - 1u) {
          sm.out[0] = k;
          sm.out[1] = o;
        }
      }
      __syncthreads();
      kstar = sm.out[0];
      istar = sm.out[1];
    } else {
      cut_by_passes<MAXPER>(sm, kv, nper, C, kmin, kmax, need, &kstar, &istar);
    }
    // emission in token order: a ballot per 64 ordinals places each taken
    // candidate, so each wave store covers one run of consecutive positions
    auto take = [&](int i) {
      const uint32_t o = uint32_t(i) * RT + tid;
      return o < C && (kv[i] > kstar || (kv[i] == kstar && o <= istar));
    };
    uint32_t off[MAXPER];
    word_offsets<MAXPER>(sm, nper, 1, take, off);
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      if (i >= nper) { JSSA_ROUNDS_END; }
      const bool t = take(i);
      const uint64_t mk = __ballot(t);
      const uint32_t pos = off[i] + uint32_t(__popcll(mk & below));
      if (t && pos < need) emit(pos, uint32_t(sm.cand[uint32_t(i) * RT + tid] >> 32));
    }
  }

  // The row's exact selection among its candidates: the k-th key K* and the
  // tie cut I*, then emit(pos, token) for each selected candidate, pos its
  // place in the ascending list (0 <= pos < kk).  Several workgroups may
  // select the same row (each emits its own part); only the `leader` resets
  // the row's state for the next call, writes n_sel and counts diagnostics.
  // REDO: the slots come from this decode's sampled threshold, so fewer than
  // k candidates mean an exact re-selection; without REDO (slots from the
  // candidate pass of an exact first-digit threshold) that cannot happen, and
  // is flagged as an error if it does.
  template <bool REDO = true, typename Emit>
  static __device__ __forceinline__ void select_row(const PipeArgs& a, int row, const RowMode& md, char* smem,
                                                    bool leader, Emit emit) {
    ResolveSmem& sm = *reinterpret_cast<ResolveSmem*>(smem);
    if (leader && threadIdx.x == 0) {  // read again only by the next call's scan
      *l_word(a, row) = 0;
      const_cast<int32_t*>(a.at.n_sel)[row] = md.kk + md.nW;
    }
    const int n_tiles_row = (md.n_cand + TS - 1) / TS;
    // the first digit's histogram is cleared while the gather's loads are in flight
    for (int i = threadIdx.x; i < 2048; i += RT) sm.hist[i] = 0u;
    if (threadIdx.x == 0) sm.n_bin = 0u;
    uint32_t kmin, kmax;
    // the sample's rank sets the expected candidates per tile: m / NSAMP of its tokens
    const int m = sample_rank(md);
    const bool wide = m * TS > 48 * NSAMP;
    uint32_t C = m == 0 ? gather_all(a, row, md.n_cand, n_tiles_row, sm, &kmin, &kmax)
                 : wide ? gather<false, 2>(a, row, n_tiles_row, sm, &kmin, &kmax)
                        : gather<false, 1>(a, row, n_tiles_row, sm, &kmin, &kmax);
    const bool fresh = C < uint32_t(md.kk);  // (m > 0) the slots are rewritten below (read back device-scope)
    if (fresh) {
      if constexpr (REDO) {
        exact_candidates(a, row, md, smem, leader);
        for (int i = threadIdx.x; i < 2048; i += RT) sm.hist[i] = 0u;
        if (threadIdx.x == 0) sm.n_bin = 0u;
        C = wide ? gather<true, 2>(a, row, n_tiles_row, sm, &kmin, &kmax)
                 : gather<true, 1>(a, row, n_tiles_row, sm, &kmin, &kmax);
      } else {
        if (threadIdx.x == 0) flag_error(a);
        return;  // uniform
      }
    }
    const uint32_t need = uint32_t(md.kk);  // 1 <= need <= C
    uint32_t kstar, istar;
    if (C <= uint32_t(kPipeCandLds / 2)) {
      cut_in_lds<kPipeCandLds / 2 / RT>(sm, C, need, kmin, kmax, emit);
    } else if (C <= uint32_t(kPipeCandLds)) {
      cut_in_lds<kPipeCandLds / RT>(sm, C, need, kmin, kmax, emit);
    } else {
      // more candidates than shared memory holds: every pass reads them in place
      if (leader && threadIdx.x == 0)
        __hip_atomic_fetch_add(a.at.queue + QW_BIG, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t* slots = a.cand + size_t(row) * a.at.t_max;
      auto global_cand = [&](uint32_t j) {
        const uint32_t tile = last_le(sm.tab, uint32_t(n_tiles_row), j);
        const uint64_t* p = slots + size_t(tile) * TS + (j - sm.tab[tile]);
        return fresh ? consume(p) : *p;
      };
      kth_cut<RT>(global_cand, C, need, true, sm.hist, sm.out, &kstar, &istar);
      const uint32_t per = (C + RT - 1) / RT;
      const uint32_t j0 = threadIdx.x * per, j1 = min(C, j0 + per);
      uint32_t mine = 0;
      for (uint32_t j = j0; j < j1; ++j) mine += passes(global_cand(j), kstar, istar);
      uint32_t total;
      uint32_t pos = block_exclusive_scan<RW>(mine, sm.scan, &total);
      for (uint32_t j = j0; j < j1; ++j) {
        const uint64_t c = global_cand(j);
        if (passes(c, kstar, istar)) {
          if (pos < need) emit(pos, uint32_t(c >> 32));
          ++pos;
        }
      }
    }
  }

  // ---- SELECT + ATTEND (second launch) ---------------------------------------------------
  // Workgroup (row, part) selects the row exactly (every part of a row does
  // the same selection; part 0 also writes n_sel and resets the row's state),
  // keeps the positions [part * chunk, (part + 1) * chunk) of the ascending
  // list plus window (and writes them to the output list), then attends over
  // them and leaves the part's partial for the row's last part to merge.  Rows with
  // nothing to choose got their list from the scan launch; their parts derive
  // their tokens from the positions.
  static constexpr int kAttnNW = kResolveThreads / 64;
  using PSmem = PortionSmem<KVT, D, G, kAttnNW, kPortionNL>;
  struct SelSmem {
    union {
      ResolveSmem rs;  // the selection (the exact re-selection overlays ScoreSmem on it)
      ScoreSmem ss;
      PSmem at;        // the attention, once the selection is done
    };
    int sidx[kPipeMaxPortion];  // the part's token indices
  };
  static_assert(sizeof(SelSmem) <= 160 * 1024, "select/attend shared memory exceeds a compute unit's 160 KiB");
  static __device__ __forceinline__ void attend_part(const PipeArgs& a, SelSmem& sm, int row, int b, int h, int part,
                                                     int cnt) {
    if (cnt <= 0) return;  // uniform over the workgroup
    attend_portion<KVT, D, G, kAttnNW, kPortionNL, true>(a.at, sm.at, sm.sidx, row, b, h, part, cnt);
  }
  // Every part of the row takes a ticket once its partial is stored (device
  // scope); the last merges the row's n_live parts.  (A merge launch of its
  // own after this one measured 1.2 us slower per 128K step.)
  static __device__ __forceinline__ void finish_row(const PipeArgs& a, int row, int n_list) {
    uint32_t* ticket = a.at.row_state + size_t(row) * kRowStateWords + RS_TICKET_ATTN;
    if (last_arrival(ticket, uint32_t(a.at.n_chunks)))
      merge_row_in_launch<D, G>(a.at, row, (n_list + a.at.chunk - 1) / a.at.chunk);
  }
  static __device__ __forceinline__ void select_attend(const PipeArgs& a, int row, int part, SelSmem& sm) {
    const int b = row / a.at.Hkv, h = row - b * a.at.Hkv;
    const RowMode md = row_mode(a, b);
    const int p0 = part * a.at.chunk;
    const int p1 = min(p0 + a.at.chunk, md.kk + md.nW);
    const int cnt = p1 > p0 ? p1 - p0 : 0;
    int32_t* out = a.at.idx + size_t(row) * a.at.idx_stride;
    if (md.select()) {
      select_row(
          a, row, md, reinterpret_cast<char*>(&sm), part == 0,
          [&](uint32_t pos, uint32_t tok) {
            if (int(pos) >= p0 && int(pos) < p1) {
              sm.sidx[int(pos) - p0] = int(tok);
              out[pos] = int(tok);
            }
          });
    }
    // positions past the selection (the window) and every position of a row
    // with nothing to choose
    for (int i = threadIdx.x; i < cnt; i += RT) {
      const int pos = p0 + i;
      if (pos >= md.kk) {
        const int tok = md.Tb - md.nW + (pos - md.kk);
        sm.sidx[i] = tok;
        if (md.select()) out[pos] = tok;
      } else if (!md.select()) {
        sm.sidx[i] = pos;
      }
    }
    __syncthreads();  // the part's list is complete; the selection's shared memory is free
    attend_part(a, sm, row, b, h, part, cnt);
    finish_row(a, row, md.kk + md.nW);
  }
  // The dense decode: part `part` of the row attends over positions
  // [part * chunk, (part + 1) * chunk) of the sequence (all of them selected).
  // (It needs no selection state: its own shared memory is the attention's
  // and the positions'.)
  struct DenseSmem {
    PortionSmem<KVT, D, G, kAttnNW, kDenseNL> at;
    int sidx[kPipeMaxPortion];
  };
  static __device__ __forceinline__ void dense_attend(const PipeArgs& a, int row, int part, DenseSmem& sm) {
    const int b = row / a.at.Hkv, h = row - b * a.at.Hkv;
    int n = a.at.seq_lens[b];
    n = n < 0 ? 0 : (n > a.at.t_max ? a.at.t_max : n);
    const int p0 = part * a.at.chunk;
    const int cnt = p0 < n ? min(a.at.chunk, n - p0) : 0;
    for (int i = threadIdx.x; i < cnt; i += RT) sm.sidx[i] = p0 + i;
    __syncthreads();
    if (cnt > 0)  // uniform over the workgroup
      attend_portion<KVT, D, G, kAttnNW, kDenseNL, true>(a.at, sm.at, sm.sidx, row, b, h, part, cnt);
    finish_row(a, row, n);
  }
  // One row's whole list from candidate slots of a previous launch (the MLA
  // decode's candidate pass): the exact cut, the ascending list and the window.
  static __device__ __forceinline__ void select_list(const PipeArgs& a, int row, char* smem) {
    const int b = row / a.at.Hkv;
    const RowMode md = row_mode(a, b);
    int32_t* out = a.at.idx + size_t(row) * a.at.idx_stride;
    if (md.select()) {
      select_row<false>(a, row, md, smem, true, [&](uint32_t pos, uint32_t tok) { out[pos] = int(tok); });
    } else {  // every candidate or none
      for (int t = threadIdx.x; t < md.kk; t += RT) out[t] = t;
      if (threadIdx.x == 0) const_cast<int32_t*>(a.at.n_sel)[row] = md.kk + md.nW;
    }
    for (int j = threadIdx.x; j < md.nW; j += RT) out[md.kk + j] = md.Tb - md.nW + j;
  }
  // The same parts over a caller's index lists (n_sel[row] entries of idx).
  static __device__ __forceinline__ void list_attend(const PipeArgs& a, int row, int part, SelSmem& sm) {
    const int b = row / a.at.Hkv, h = row - b * a.at.Hkv;
    int n = a.at.n_sel[row];
    n = n < 0 ? 0 : (n > a.at.idx_stride ? a.at.idx_stride : n);
    const int p0 = part * a.at.chunk;
    const int cnt = p0 < n ? min(a.at.chunk, n - p0) : 0;
    const int32_t* src = a.at.idx + size_t(row) * a.at.idx_stride + p0;
    for (int i = threadIdx.x; i < cnt; i += RT) sm.sidx[i] = src[i];
    __syncthreads();
    attend_part(a, sm, row, b, h, part, cnt);
    finish_row(a, row, n);
  }
};

// Scan launch: workgroup r < n_rows first samples row r (when the grid
// covers every row; the grid never exceeds the resident workgroups, and the
// samples wait for nothing, so every row's threshold gets published), then
// each workgroup takes its share of the split of the score work.  A score range waits for its row's threshold only after its
// first scan, under a deadline (a missing threshold is flagged, never waited
// for forever).
template <int KPT, int R, int GE, int D, int G, int KVT>
__global__ __launch_bounds__(256, 3) void scan_kernel(PipeArgs a) {
  using Pp = Pipe<KPT, R, GE, D, G, KVT>;
  __shared__ __align__(16) char smem[Pp::kSmemScan];
  __shared__ typename Pp::FlatSmem fs;
  const uint64_t deadline = wall_clock64() + a.spin_ticks;
  if (a.samples_in_scan && int(blockIdx.x) < a.n_rows) {  // one sample per workgroup at most
    Pp::sample(a, blockIdx.x, *reinterpret_cast<typename Pp::SampleSmem*>(smem));
    __syncthreads();
  }
  Pp::score_split(a, smem, fs, deadline);
}

// More rows than the scan's resident workgroups: the samples (and the
// step's appends) run in a launch of their own first, one row per workgroup.
template <int KPT, int R, int GE, int D, int G, int KVT>
__global__ __launch_bounds__(256, 3) void sample_kernel(PipeArgs a) {
  using Pp = Pipe<KPT, R, GE, D, G, KVT>;
  __shared__ __align__(16) char smem[sizeof(typename Pp::SampleSmem)];
  Pp::sample(a, blockIdx.x, *reinterpret_cast<typename Pp::SampleSmem*>(smem));
}

// Workgroup i of the select/attend launches runs on XCD i mod 8: the parts of
// a row are placed on one XCD, so the row's candidates, read by every part,
// come from that XCD's L2 after the first read.  False for the padding
// workgroups of the last rows.
__device__ __forceinline__ bool part_of(const PipeArgs& a, int i, int* row, int* part) {
  const int x = i & 7, j = i >> 3;
  *row = x + 8 * (j / a.at.n_chunks);
  *part = j % a.at.n_chunks;
  return *row < a.n_rows;
}

// Select + attend launch: one workgroup per (row, part of its list).
template <int KPT, int R, int GE, int D, int G, int KVT>
__global__ __launch_bounds__(kResolveThreads, 1) void select_attend_kernel(PipeArgs a) {
  using Pp = Pipe<KPT, R, GE, D, G, KVT>;
  __shared__ __align__(16) char smem[sizeof(typename Pp::SelSmem)];
  int row, part;
  if (!part_of(a, blockIdx.x, &row, &part)) return;
  Pp::select_attend(a, row, part, *reinterpret_cast<typename Pp::SelSmem*>(smem));
}

// The dense decode's parts (the decode's attention over every position).
template <int KPT, int R, int GE, int D, int G, int KVT>
__global__ __launch_bounds__(kResolveThreads, 1) void dense_attend_kernel(PipeArgs a) {
  using Pp = Pipe<KPT, R, GE, D, G, KVT>;
  __shared__ __align__(16) char smem[sizeof(typename Pp::DenseSmem)];
  int row, part;
  if (!part_of(a, blockIdx.x, &row, &part)) return;
  Pp::dense_attend(a, row, part, *reinterpret_cast<typename Pp::DenseSmem*>(smem));
}

// Selection only, one workgroup per row (the MLA decode's rows).
template <int KPT, int R, int GE, int D, int G, int KVT>
__global__ __launch_bounds__(kResolveThreads, 1) void select_only_kernel(PipeArgs a) {
  using Pp = Pipe<KPT, R, GE, D, G, KVT>;
  __shared__ __align__(16) char smem[sizeof(typename Pp::SelSmem)];
  Pp::select_list(a, blockIdx.x, smem);
}

// Attention over caller lists: the same parts and arithmetic.
template <int KPT, int R, int GE, int D, int G, int KVT>
__global__ __launch_bounds__(kResolveThreads, 1) void list_attend_kernel(PipeArgs a) {
  using Pp = Pipe<KPT, R, GE, D, G, KVT>;
  __shared__ __align__(16) char smem[sizeof(typename Pp::SelSmem)];
  int row, part;
  if (!part_of(a, blockIdx.x, &row, &part)) return;
  Pp::list_attend(a, row, part, *reinterpret_cast<typename Pp::SelSmem*>(smem));
}


// ---- host side ------------------------------------------------------------------------------
// Shapes with a fused build: (kv dtype, kp dtype, d, rank, G).  Others run the staged launches.
struct PipeShape {
  int kv, kp, d, r, g;
};
static const PipeShape kPipeShapes[] = {
    {JSSA_BF16, JSSA_BF16, 128, 32, 4},     {JSSA_BF16, JSSA_BF16, 128, 64, 1},
    {JSSA_BF16, JSSA_BF16, 64, 16, 4},      {JSSA_F32, JSSA_F32, 64, 16, 4},
    {JSSA_F32, JSSA_F32, 128, 32, 2},       {JSSA_BF16, JSSA_FP8_E4M3, 128, 32, 4},
    {JSSA_BF16, JSSA_FP8_E4M3, 128, 64, 1},
};

static int scan_tile_tokens(int dt, int r) {
  const int per16 = dt == JSSA_FP8_E4M3 ? 16 : dt == JSSA_BF16 ? 8 : 4;
  const int per_iter = 4 * (64 / (r / per16)) * JSSA_SCORE_UNROLL;
  return kPipeTileTokens > 2 * per_iter ? kPipeTileTokens : 2 * per_iter;  // Pipe::TS
}

bool pipeline_layout(const jssa_desc& d, int* ts, int* n_tiles, int* chunk) {
  const int G = d.n_q_heads / d.n_kv_heads;
  bool ok = false;
  for (const PipeShape& s : kPipeShapes)
    ok |= (d.kv_dtype == s.kv && d.kp_dtype == s.kp && d.d_k == s.d && d.rank == s.r && G == s.g);
  if (!ok || d.layout != JSSA_LAYOUT_GQA) return false;
  *ts = scan_tile_tokens(d.kp_dtype, d.rank);
  *n_tiles = (d.t_max + *ts - 1) / *ts;
  // the select/attend parts of a row: about kPipePartTarget workgroups in all,
  // at most kPipeMaxPortion list positions each (a function of the descriptor
  // only, so results do not depend on the device)
  const int64_t n_max = int64_t(d.topk) + d.window;
  const int64_t rows = int64_t(d.batch) * d.n_kv_heads;
  int64_t parts = (kPipePartTarget + rows - 1) / rows;
  if (parts > kPipeMaxParts) parts = kPipeMaxParts;
  const int64_t need = (n_max + kPipeMaxPortion - 1) / kPipeMaxPortion;
  if (parts < need) parts = need;
  if (parts > kPipeMaxParts || n_max < 1) return false;
  int64_t c = (n_max + parts - 1) / parts;
  c = (c + 63) / 64 * 64;
  *chunk = int(c);  // list positions per part; ceil(n_max / chunk) <= kPipeMaxParts parts
  return *n_tiles <= kPipeMaxTiles;
}

bool dense_pipe_layout(const jssa_desc& d, int* chunk, int* n_chunks) {
  const int G = d.n_q_heads / d.n_kv_heads;
  bool ok = false;
  for (const PipeShape& s : kPipeShapes)
    ok |= (d.kv_dtype == s.kv && d.kp_dtype == s.kp && d.d_k == s.d && d.rank == s.r && G == s.g);
  if (!ok || d.layout != JSSA_LAYOUT_GQA || d.t_max < 1) return false;
  // parts of at most kPipeMaxPortion positions, and about kPipePartTarget
  // workgroups in all when the rows are short (a cache of a few thousand
  // positions, such as the packed rows of the gather-then-attend baseline,
  // gets the sparse decode's part size instead of one workgroup per row)
  const int64_t rows = int64_t(d.batch) * d.n_kv_heads;
  const int64_t parts = (kPipePartTarget + rows - 1) / rows;
  int64_t c = (int64_t(d.t_max) + parts - 1) / parts;
  c = (c + 63) / 64 * 64;
  if (c > kPipeMaxPortion) c = kPipeMaxPortion;
  *chunk = int(c);
  *n_chunks = int((d.t_max + c - 1) / c);
  return true;
}

// Ticks of the device wall clock in 4 seconds (the bound on every wait).
static uint64_t wait_ticks() {
  static uint64_t ticks[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 400000000ull;
  if (ticks[dev] == 0) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz < 1) khz = 100000;
    ticks[dev] = uint64_t(khz) * 1000ull * 4ull;
  }
  return ticks[dev];
}

// Compute units of the current device (cached per device).
static int compute_units() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Scan workgroups resident per compute unit (cached per device and kernel).
template <int KPT, int R, int GE, int D, int G, int KVT>
static int scan_per_cu() {
  static int per_cu[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (per_cu[dev] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, scan_kernel<KPT, R, GE, D, G, KVT>, 256, 0) != hipSuccess ||
        n < 1)
      n = 1;
#if JSSA_PIPE_PER_CU > 0
    if (n > JSSA_PIPE_PER_CU) n = JSSA_PIPE_PER_CU;
#endif
    per_cu[dev] = n;
  }
  return per_cu[dev];
}

template <int KPT, int R, int GE, int D, int G, int KVT>
static hipError_t launch_pipe_t(PipeArgs a, void* const* ev, hipStream_t s) {
  using Pp = Pipe<KPT, R, GE, D, G, KVT>;
  if (Pp::TS != a.ts || a.at.chunk % 64 != 0 || a.at.chunk > kPipeMaxPortion || a.at.n_chunks > kPipeMaxParts)
    return hipErrorInvalidValue;
  if (a.attend_only) {  // caller-provided index lists: the attention parts (with their merge) only
    hipLaunchKernelGGL((list_attend_kernel<KPT, R, GE, D, G, KVT>), dim3(a.n_attn), dim3(kResolveThreads), 0, s, a);
    return hipGetLastError();
  }
  // At most one workgroup per resident slot: the samples, then as many score
  // workgroups as the closed-form split of rows of t_max tokens uses (the
  // split of shorter or ragged rows adapts to whatever grid it gets).
  const int resident = scan_per_cu<KPT, R, GE, D, G, KVT>() * compute_units();
  const int n_tiles_max = (a.at.t_max + Pp::TS - 1) / Pp::TS;
  int grid = resident;
  if (resident >= 2 * a.n_rows) {
    const int per_row = (resident - a.n_rows) / a.n_rows;
    const int it = (n_tiles_max + per_row - 1) / per_row, runs = (n_tiles_max + it - 1) / it;
    grid = a.n_rows * (1 + runs);
  } else {
    const int64_t useful = int64_t(a.n_rows) * (1 + n_tiles_max);
    if (useful < grid) grid = int(useful);
  }
  a.samples_in_scan = a.n_rows <= grid;
  auto mark = [&](int i) { return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess; };
  hipError_t e = hipSuccess;
  if (!a.samples_in_scan) {
    hipLaunchKernelGGL((sample_kernel<KPT, R, GE, D, G, KVT>), dim3(a.n_rows), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev) {  // events [0] and [1] take the scan kernel's own start and end
    hipExtLaunchKernelGGL((scan_kernel<KPT, R, GE, D, G, KVT>), dim3(grid), dim3(256), 0, s,
                          static_cast<hipEvent_t>(ev[0]), static_cast<hipEvent_t>(ev[1]), 0u, a);
  } else {
    hipLaunchKernelGGL((scan_kernel<KPT, R, GE, D, G, KVT>), dim3(grid), dim3(256), 0, s, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((select_attend_kernel<KPT, R, GE, D, G, KVT>), dim3(a.n_attn), dim3(kResolveThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(2)) != hipSuccess) return e;
  return mark(3);
}

template <int KVT, int KPT, int D, int R, int G>
static hipError_t launch_pipe_reduce(const PipeArgs& a, bool mean, void* const* ev, hipStream_t s) {
  if (mean) return launch_pipe_t<KPT, R, 1, D, G, KVT>(a, ev, s);
  return launch_pipe_t<KPT, R, G, D, G, KVT>(a, ev, s);
}

static hipError_t pipeline_impl(const jssa_desc& d, const void* q, const float* P, const void* kp,
                                const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                                float* lse, int32_t* idx, int32_t* n_sel, char* ws_base, const Workspace& ws,
                                const NewToken* nt, void* const* ev, bool attend_only, hipStream_t s) {
  if (!ws.pipe) return hipErrorInvalidValue;
  PipeArgs a{};
  a.attend_only = attend_only;
  if (nt) {
    a.k_new = nt->k_new; a.v_new = nt->v_new; a.pos = nt->pos;
    a.k_w = nt->k_cache; a.v_w = nt->v_cache; a.kp_w = nt->kp_cache;
  }
  AttnArgs& at = a.at;
  at.q = q; at.k = k_cache; at.v = v_cache; at.idx = idx; at.n_sel = n_sel; at.seq_lens = seq_lens;
  at.out = out; at.lse = lse;
  at.part_acc = reinterpret_cast<float*>(ws_base + ws.part_acc);
  at.part_ml = reinterpret_cast<float*>(ws_base + ws.part_ml);
  at.row_state = reinterpret_cast<uint32_t*>(ws_base + ws.row_state);
  at.queue = reinterpret_cast<uint32_t*>(ws_base + ws.queue);
  at.Hq = d.n_q_heads; at.Hkv = d.n_kv_heads; at.t_max = d.t_max;
  at.idx_stride = d.topk + d.window; at.chunk = ws.pipe_chunk; at.n_chunks = ws.pipe_n_chunks;
  at.out_dtype = d.out_dtype; at.qscale = d.scale * kLog2e;
  at.n_resolve = 0; at.attend = 1;
  a.P = P; a.kp = kp;
  a.cand = reinterpret_cast<uint64_t*>(ws_base + ws.cand);
  a.qp_pub = reinterpret_cast<float*>(ws_base + ws.pipe_qp);
  a.tile_cnt = reinterpret_cast<uint32_t*>(ws_base + ws.tile_cnt);
  a.G = d.n_q_heads / d.n_kv_heads; a.d_k = d.d_k; a.topk = d.topk; a.window = d.window;
  a.q_dtype = d.kv_dtype; a.ts = ws.pipe_ts; a.n_tiles = ws.pipe_tiles;
  a.n_rows = d.batch * d.n_kv_heads;
  a.n_attn = 8 * ((a.n_rows + 7) / 8) * ws.pipe_n_chunks;  // (row, part) workgroups, rows padded to the 8 XCDs
  a.spin_ticks = wait_ticks();
  const int G = a.G;
  const bool mean = d.reduce == JSSA_REDUCE_MEAN;
  if (d.kv_dtype == JSSA_BF16 && d.kp_dtype == JSSA_FP8_E4M3) {
    if (d.d_k == 128 && d.rank == 32 && G == 4) return launch_pipe_reduce<1, 2, 128, 32, 4>(a, mean, ev, s);
    if (d.d_k == 128 && d.rank == 64 && G == 1) return launch_pipe_reduce<1, 2, 128, 64, 1>(a, mean, ev, s);
  } else if (d.kv_dtype == JSSA_BF16) {
    if (d.d_k == 128 && d.rank == 32 && G == 4) return launch_pipe_reduce<1, 1, 128, 32, 4>(a, mean, ev, s);
    if (d.d_k == 128 && d.rank == 64 && G == 1) return launch_pipe_reduce<1, 1, 128, 64, 1>(a, mean, ev, s);
    if (d.d_k == 64 && d.rank == 16 && G == 4) return launch_pipe_reduce<1, 1, 64, 16, 4>(a, mean, ev, s);
  } else {
    if (d.d_k == 64 && d.rank == 16 && G == 4) return launch_pipe_reduce<0, 0, 64, 16, 4>(a, mean, ev, s);
    if (d.d_k == 128 && d.rank == 32 && G == 2) return launch_pipe_reduce<0, 0, 128, 32, 2>(a, mean, ev, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pipeline(const jssa_desc& d, const void* q, const float* P, const void* kp,
                           const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                           float* lse, int32_t* idx, int32_t* n_sel, char* ws_base, const Workspace& ws,
                           const NewToken* nt, void* const* ev, hipStream_t s) {
  return pipeline_impl(d, q, P, kp, k_cache, v_cache, seq_lens, out, lse, idx, n_sel, ws_base, ws, nt, ev, false, s);
}

// The exact selection of every row from the candidate pass's slots (per
// kSubTile tokens, a count per tile, from a first-digit threshold that admits
// at least k keys), with the fused decode's selection: one 1024-thread
// workgroup per row.  Any fused shape's selection code serves (it reads only
// keys and token indices); this one has kSubTile-token tiles.
hipError_t launch_select_rows(const jssa_desc& d, const int32_t* seq_lens, int32_t* idx, int32_t* n_sel,
                              char* ws_base, const Workspace& ws, hipStream_t s) {
  using Pp = Pipe<1, 32, 4, 128, 4, 1>;
  static_assert(Pp::TS == kSubTile, "the candidate pass's tiles");
  PipeArgs a{};
  AttnArgs& at = a.at;
  at.seq_lens = seq_lens; at.idx = idx; at.n_sel = n_sel;
  at.Hkv = d.n_kv_heads; at.t_max = d.t_max; at.idx_stride = d.topk + d.window;
  at.queue = reinterpret_cast<uint32_t*>(ws_base + ws.queue);
  at.row_state = reinterpret_cast<uint32_t*>(ws_base + ws.row_state);
  a.cand = reinterpret_cast<uint64_t*>(ws_base + ws.cand);
  a.tile_cnt = reinterpret_cast<uint32_t*>(ws_base + ws.tile_cnt);
  a.n_tiles = ws.n_sel_tiles * (kSelTile / kSubTile);  // the counts' row stride
  a.topk = d.topk; a.window = d.window; a.ts = kSubTile;
  a.n_rows = d.batch * d.n_kv_heads;
  if ((d.t_max + kSubTile - 1) / kSubTile > kPipeMaxTiles) return hipErrorInvalidValue;
  hipLaunchKernelGGL((select_only_kernel<1, 32, 4, 128, 4, 1>), dim3(a.n_rows), dim3(kResolveThreads), 0, s, a);
  return hipGetLastError();
}

// The dense decode on the fused shapes: every position of every row, in
// parts of kPipeMaxPortion positions, with the decode's attention and
// in-launch merge (one 1024-thread workgroup per part, a row's parts on one
// XCD).
template <int KPT, int R, int D, int G, int KVT>
static hipError_t launch_dense_t(const PipeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((dense_attend_kernel<KPT, R, G, D, G, KVT>), dim3(a.n_attn), dim3(kResolveThreads), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_pipe_dense(const jssa_desc& d, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, void* out, float* lse, char* ws_base, const Workspace& ws,
                             hipStream_t s) {
  if (!ws.pipe || ws.pipe_chunk < 1 || ws.pipe_chunk > kPipeMaxPortion) return hipErrorInvalidValue;
  PipeArgs a{};
  AttnArgs& at = a.at;
  at.q = q; at.k = k_cache; at.v = v_cache; at.seq_lens = seq_lens; at.out = out; at.lse = lse;
  at.part_acc = reinterpret_cast<float*>(ws_base + ws.part_acc);
  at.part_ml = reinterpret_cast<float*>(ws_base + ws.part_ml);
  at.row_state = reinterpret_cast<uint32_t*>(ws_base + ws.row_state);
  at.queue = reinterpret_cast<uint32_t*>(ws_base + ws.queue);
  at.Hq = d.n_q_heads; at.Hkv = d.n_kv_heads; at.t_max = d.t_max;
  at.chunk = ws.pipe_chunk; at.n_chunks = ws.pipe_n_chunks;
  at.out_dtype = d.out_dtype; at.qscale = d.scale * kLog2e;
  at.attend = 1;
  a.G = d.n_q_heads / d.n_kv_heads; a.d_k = d.d_k;
  a.n_rows = d.batch * d.n_kv_heads;
  a.n_attn = 8 * ((a.n_rows + 7) / 8) * ws.pipe_n_chunks;
  a.spin_ticks = wait_ticks();
  // the attention depends on the K/V type, d and G only: one instantiation each
  const int G = a.G;
  if (d.kv_dtype == JSSA_BF16) {
    if (d.d_k == 128 && G == 4) return launch_dense_t<1, 32, 128, 4, 1>(a, s);
    if (d.d_k == 128 && G == 1) return launch_dense_t<1, 64, 128, 1, 1>(a, s);
    if (d.d_k == 64 && G == 4) return launch_dense_t<1, 16, 64, 4, 1>(a, s);
  } else {
    if (d.d_k == 64 && G == 4) return launch_dense_t<0, 16, 64, 4, 0>(a, s);
    if (d.d_k == 128 && G == 2) return launch_dense_t<0, 32, 128, 2, 0>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pipe_attend(const jssa_desc& d, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* idx, const int32_t* n_sel, void* out, float* lse, char* ws_base,
                              const Workspace& ws, hipStream_t s) {
  return pipeline_impl(d, q, nullptr, nullptr, k_cache, v_cache, nullptr, out, lse, const_cast<int32_t*>(idx),
                       const_cast<int32_t*>(n_sel), ws_base, ws, nullptr, nullptr, true, s);
}

}  // namespace jssa
