// Subspace score scan (JSSA summary Figure 1, sections 3.1 and E.1): every
// candidate token of every (sequence, KV head) is scored against the
// projected queries of the head's group, reading the projected-key cache once
// with coalesced 16-byte loads.  Optionally builds the first radix digit
// histogram of the scores for selection, so that selection needs no extra
// pass over the scores for it.
#include "jssa_device.hpp"
#include "jssa_internal.hpp"
#include "score_core.hpp"
#include "select_common.hpp"

namespace jssa {

struct ScoreArgs {
  const void* q;
  const float* P;
  const void* kp;
  const int32_t* seq_lens;
  float* scores;
  uint32_t* hist1;      // null: no histogram
  uint32_t* row_state;
  int Hq, Hkv, G, d_k, t_max, topk, window, q_dtype;
};

// One workgroup (4 waves) per kScoreTile candidate tokens of one (b, h) row.
// The scores of a step come from score_loads (score_core.hpp): on the matrix
// cores for bf16 keys of rank 32 or 64, with DPP dot products otherwise.
// Loads are double-buffered: the next step's 16-byte vectors are in flight
// while the current ones are scored.  GE = G for the group max, 1 for the mean.
template <int KPT, int R, int GE>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  using S = ScanShape<KPT, R>;
  constexpr int EB = S::EB, U = S::U, PER_ITER = S::PER_ITER;

  __shared__ uint32_t s_hist[kDigit1Bins];
  __shared__ float s_q[8 * 128];
  __shared__ float s_part[512];
  __shared__ float s_qp[8 * 64];
  __shared__ uint32_t s_scan[8];
  __shared__ uint32_t s_out[2];

  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int row = b * a.Hkv + h;
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  const int t0 = tile * kScoreTile;
  if (t0 >= n_cand) return;
  const bool do_hist = a.hist1 != nullptr && a.topk > 0 && a.topk < n_cand;
  const int t_end = min(t0 + kScoreTile, n_cand);
  const char* kp_row = reinterpret_cast<const char*>(a.kp) + size_t(row) * a.t_max * R * EB;
  float* srow = a.scores + size_t(row) * a.t_max;

  // Loads are issued without per-lane branches (tokens past the end re-read the
  // last candidate and are discarded), so the compiler can keep the next
  // step's loads in flight while the current step is scored.
  auto load_step = [&](int base, uint4 (&v)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tok = min(base + slot_token<KPT, R>(u), t_end - 1);
      v[u] = load16_nt(kp_row + size_t(tok) * R * EB + slot_byte<KPT, R>(u));
    }
  };
  uint4 cur[U];
  load_step(t0, cur);  // first loads go out before the query projection

  if (do_hist)
    for (int i = threadIdx.x; i < kDigit1Bins; i += 256) s_hist[i] = 0u;
  const int G = a.G;
  project_group_query<R>(a.q, a.q_dtype, a.P, a.Hq, a.d_k, G, b, h, s_q, s_part, s_qp);

  QFrag<KPT, R, GE> qf;
  load_qfrag<KPT, R, GE>([&](int i) { return s_qp[i]; }, G, qf);

  for (int base = t0; base < t_end; base += PER_ITER) {
    uint4 nxt[U];
    load_step(base + PER_ITER, nxt);
    score_loads<KPT, R, GE>(cur, qf, G, [&](int toff, float best) {
      const int tok = base + toff;
      if (tok < t_end) {
        srow[tok] = best;
        if (do_hist) atomicAdd(&s_hist[score_key(best) >> (32 - kDigit1Bits)], 1u);
      }
    });
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }

  if (!do_hist) return;
  __syncthreads();
  uint32_t* g_hist = a.hist1 + size_t(row) * kDigit1Bins;
  for (int i = threadIdx.x; i < kDigit1Bins; i += 256) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(&g_hist[i], c);
  }
  uint32_t* g_state = a.row_state + size_t(row) * kRowStateWords;
  const uint32_t n_tiles = uint32_t((n_cand + kScoreTile - 1) / kScoreTile);
  if (!last_arrival(&g_state[RS_TICKET_SCORE], n_tiles)) return;
  finish_first_digit(g_hist, g_state, s_hist, s_scan, s_out, uint32_t(a.topk));
}

// First-digit histogram of caller-provided fp32 scores (the stand-alone
// selection entry point), one workgroup per kSelTile keys of a row.
struct HistArgs {
  const float* scores;
  const int32_t* seq_lens;
  uint32_t* hist1;
  uint32_t* row_state;
  int Hkv, t_max, topk, window;
};

__global__ __launch_bounds__(256) void hist_kernel(HistArgs a) {
  __shared__ uint32_t s_hist[kDigit1Bins];
  __shared__ uint32_t s_scan[8];
  __shared__ uint32_t s_out[2];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int row = b * a.Hkv + h;
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  const int t0 = tile * kSelTile;
  if (t0 >= n_cand || a.topk <= 0 || a.topk >= n_cand) return;
  for (int i = threadIdx.x; i < kDigit1Bins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  const float* srow = a.scores + size_t(row) * a.t_max;
  const int t_end = min(t0 + kSelTile, n_cand);
  constexpr int KPT_ = kSelTile / 256;
  float v[KPT_];
#pragma unroll
  for (int i = 0; i < KPT_; ++i) v[i] = srow[min(t0 + i * 256 + int(threadIdx.x), t_end - 1)];
#pragma unroll
  for (int i = 0; i < KPT_; ++i)
    if (t0 + i * 256 + int(threadIdx.x) < t_end) atomicAdd(&s_hist[score_key(v[i]) >> (32 - kDigit1Bits)], 1u);
  __syncthreads();
  uint32_t* g_hist = a.hist1 + size_t(row) * kDigit1Bins;
  for (int i = threadIdx.x; i < kDigit1Bins; i += 256) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(&g_hist[i], c);
  }
  uint32_t* g_state = a.row_state + size_t(row) * kRowStateWords;
  const uint32_t n_tiles = uint32_t((n_cand + kSelTile - 1) / kSelTile);
  if (!last_arrival(&g_state[RS_TICKET_SCORE], n_tiles)) return;
  finish_first_digit(g_hist, g_state, s_hist, s_scan, s_out, uint32_t(a.topk));
}

// ---- launchers ----------------------------------------------------------------------
template <int KPT, int R, int GE>
static hipError_t launch_score_t(const ScoreArgs& args, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((score_kernel<KPT, R, GE>), grid, dim3(256), 0, s, args);
  return hipGetLastError();
}

template <int KPT, int R>
static hipError_t dispatch_ge(const ScoreArgs& args, int ge, dim3 grid, hipStream_t s) {
  switch (ge) {
    case 1: return launch_score_t<KPT, R, 1>(args, grid, s);
    case 2: return launch_score_t<KPT, R, 2>(args, grid, s);
    case 4: return launch_score_t<KPT, R, 4>(args, grid, s);
    case 8: return launch_score_t<KPT, R, 8>(args, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int KPT>
static hipError_t dispatch_r(const ScoreArgs& args, int r, int ge, dim3 grid, hipStream_t s) {
  switch (r) {
    case 16: return dispatch_ge<KPT, 16>(args, ge, grid, s);
    case 32: return dispatch_ge<KPT, 32>(args, ge, grid, s);
    case 64: return dispatch_ge<KPT, 64>(args, ge, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score(const jssa_desc& d, const void* q, const float* P, const void* kp,
                        const int32_t* seq_lens, float* scores, char* ws_base, const Workspace& ws,
                        hipStream_t s) {
  ScoreArgs a;
  a.q = q; a.P = P; a.kp = kp; a.seq_lens = seq_lens; a.scores = scores;
  a.hist1 = ws_base ? reinterpret_cast<uint32_t*>(ws_base + ws.hist1) : nullptr;
  a.row_state = ws_base ? reinterpret_cast<uint32_t*>(ws_base + ws.row_state) : nullptr;
  a.Hq = d.n_q_heads; a.Hkv = d.n_kv_heads; a.G = d.n_q_heads / d.n_kv_heads;
  a.d_k = d.d_k; a.t_max = d.t_max; a.topk = d.topk; a.window = d.window; a.q_dtype = d.kv_dtype;
  const int ge = (d.reduce == JSSA_REDUCE_MEAN) ? 1 : a.G;
  dim3 grid((d.t_max + kScoreTile - 1) / kScoreTile, d.n_kv_heads, d.batch);
  if (d.kp_dtype == JSSA_FP8_E4M3) {  // matrix-core shapes only
    if (d.rank == 32) return dispatch_ge<2, 32>(a, ge, grid, s);
    if (d.rank == 64) return dispatch_ge<2, 64>(a, ge, grid, s);
    return hipErrorInvalidValue;
  }
  if (d.kp_dtype == JSSA_BF16) return dispatch_r<1>(a, d.rank, ge, grid, s);
  return dispatch_r<0>(a, d.rank, ge, grid, s);
}

hipError_t launch_hist(const jssa_desc& d, const float* scores, const int32_t* seq_lens,
                       char* ws_base, const Workspace& ws, hipStream_t s) {
  HistArgs a;
  a.scores = scores; a.seq_lens = seq_lens;
  a.hist1 = reinterpret_cast<uint32_t*>(ws_base + ws.hist1);
  a.row_state = reinterpret_cast<uint32_t*>(ws_base + ws.row_state);
  a.Hkv = d.n_kv_heads; a.t_max = d.t_max; a.topk = d.topk; a.window = d.window;
  dim3 grid((d.t_max + kSelTile - 1) / kSelTile, d.n_kv_heads, d.batch);
  hipLaunchKernelGGL(hist_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace jssa
