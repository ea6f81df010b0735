// Exact per-(sequence, KV head) top-k selection over fp32 scores (JSSA
// summary Figure 1 and section 3.1; ties to the lower token index).
//
// Radix select on order-preserving uint32 keys:
//   digit 1 (bits 31..20): histogram built by the score kernel (or by
//     hist_kernel), threshold bin D1 found by the row's last workgroup;
//   select_kernel: every workgroup counts its keys above D1 and appends the
//     keys in bin D1 to a per-row candidate list; the row's last workgroup
//     resolves the exact k-th key K* (digits 2 and 3 over the candidates),
//     the index cut I* among keys equal to K* (ties to the lower index), and
//     the output offset of every tile;
//   emit_kernel: every workgroup writes its selected indices in ascending
//     token order at its tile's offset, then the window follows.
#include "jssa_device.hpp"
#include "jssa_internal.hpp"
#include "select_common.hpp"

namespace jssa {

struct SelArgs {
  const float* scores;
  const int32_t* seq_lens;
  int32_t* idx;
  int32_t* n_sel;
  uint32_t* row_state;
  uint32_t* hist2;
  uint32_t* tile_gt;
  uint32_t* tile_off;
  uint64_t* cand;  // (index << 32) | key
  int Hkv, t_max, topk, window, n_sel_tiles;
};

__device__ __forceinline__ bool is_selected(uint32_t key, int t, uint32_t kstar, uint32_t istar) {
  return key > kstar || (key == kstar && uint32_t(t) <= istar);
}

constexpr int kDigit2Bins = 4096;  // key bits 19..8

__global__ __launch_bounds__(256) void select_kernel(SelArgs a) {
  __shared__ uint64_t s_cand[kSelTile];        // this tile's candidates; later per-tile counts
  __shared__ uint32_t s_hist[kDigit2Bins];     // digit-2 histogram; later digit 3 / index digits
  __shared__ uint32_t s_scan[8];
  __shared__ uint32_t s_out[2];
  __shared__ uint32_t s_n, s_gt, s_base;

  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int row = b * a.Hkv + h;
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  if (a.topk <= 0 || a.topk >= n_cand) return;
  const int t0 = tile * kSelTile;
  if (t0 >= n_cand) return;
  const int t_end = min(t0 + kSelTile, n_cand);
  uint32_t* g_state = a.row_state + size_t(row) * kRowStateWords;
  uint32_t* g_hist2 = a.hist2 + size_t(row) * kDigit2Bins;
  const uint32_t D1 = g_state[RS_D1];
  const float* srow = a.scores + size_t(row) * a.t_max;

  for (int i = threadIdx.x; i < kDigit2Bins; i += 256) s_hist[i] = 0u;
  if (threadIdx.x == 0) { s_n = 0u; s_gt = 0u; }
  __syncthreads();
  uint32_t gt = 0;
  for (int t = t0 + threadIdx.x; t < t_end; t += 256) {
    const uint32_t key = score_key(srow[t]);
    const uint32_t dg = key >> (32 - kDigit1Bits);
    gt += (dg > D1);
    if (dg == D1) {
      const uint32_t slot = atomicAdd(&s_n, 1u);
      s_cand[slot] = (uint64_t(uint32_t(t)) << 32) | key;
      atomicAdd(&s_hist[(key >> 8) & 0xfffu], 1u);
    }
  }
  atomicAdd(&s_gt, gt);
  __syncthreads();
  if (threadIdx.x == 0) {
    s_base = atomicAdd(&g_state[RS_CAND_COUNT], s_n);
    publish(&a.tile_gt[size_t(row) * a.n_sel_tiles + tile], s_gt);
  }
  for (int i = threadIdx.x; i < kDigit2Bins; i += 256) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(&g_hist2[i], c);
  }
  __syncthreads();
  uint64_t* clist = a.cand + size_t(row) * a.t_max;
  for (uint32_t j = threadIdx.x; j < s_n; j += 256) publish(&clist[s_base + j], s_cand[j]);

  const uint32_t n_tiles = uint32_t((n_cand + kSelTile - 1) / kSelTile);
  if (!last_arrival(&g_state[RS_TICKET_CAND], n_tiles)) return;

  // ---- resolution by the row's last workgroup ------------------------------------
  const uint32_t C = consume(&g_state[RS_CAND_COUNT]);
  const uint32_t need1 = g_state[RS_NEED1];

  // digit 2 (key bits 19..8) from the histogram every workgroup contributed to
  for (int i = threadIdx.x; i < kDigit2Bins; i += 256) {
    s_hist[i] = consume(&g_hist2[i]);
    publish(&g_hist2[i], 0u);  // zero for the next call
  }
  __syncthreads();
  find_bin_from_top<kDigit2Bins / 256>(s_hist, need1, s_scan, s_out);
  const uint32_t D2 = s_out[0];
  const uint32_t need2 = need1 - s_out[1];
  __syncthreads();

  // digit 3 (key bits 7..0) over the candidates in bin D2
  if (threadIdx.x < 256) s_hist[threadIdx.x] = 0u;
  __syncthreads();
  for (uint32_t j = threadIdx.x; j < C; j += 256) {
    const uint32_t key = uint32_t(consume(&clist[j]));
    if (((key >> 8) & 0xfffu) == D2) atomicAdd(&s_hist[key & 0xffu], 1u);
  }
  __syncthreads();
  find_bin_from_top<1>(s_hist, need2, s_scan, s_out);
  const uint32_t D3 = s_out[0];
  const uint32_t m_ties = need2 - s_out[1];  // keys equal to K* still to take (lowest indices)
  const uint32_t n_eq = s_hist[D3];
  const uint32_t kstar = (D1 << 20) | (D2 << 8) | D3;
  __syncthreads();

  uint32_t istar = 0x7fffffffu;
  if (m_ties < n_eq) {
    // the m_ties-th smallest index among keys equal to K*: index bits 23..12, then 11..0
    for (int i = threadIdx.x; i < 4096; i += 256) s_hist[i] = 0u;
    __syncthreads();
    for (uint32_t j = threadIdx.x; j < C; j += 256) {
      const uint64_t c = consume(&clist[j]);
      if (uint32_t(c) == kstar) atomicAdd(&s_hist[uint32_t(c >> 32) >> 12], 1u);
    }
    __syncthreads();
    find_bin_from_bottom<16>(s_hist, m_ties, s_scan, s_out);
    const uint32_t E1 = s_out[0];
    const uint32_t m2 = m_ties - s_out[1];
    __syncthreads();
    for (int i = threadIdx.x; i < 4096; i += 256) s_hist[i] = 0u;
    __syncthreads();
    for (uint32_t j = threadIdx.x; j < C; j += 256) {
      const uint64_t c = consume(&clist[j]);
      const uint32_t t = uint32_t(c >> 32);
      if (uint32_t(c) == kstar && (t >> 12) == E1) atomicAdd(&s_hist[t & 0xfffu], 1u);
    }
    __syncthreads();
    find_bin_from_bottom<16>(s_hist, m2, s_scan, s_out);
    istar = (E1 << 12) | s_out[0];
    __syncthreads();
  }

  // per-tile selected counts -> exclusive offsets
  uint32_t* s_cnt = reinterpret_cast<uint32_t*>(s_cand);  // kMaxSelTiles words fit in s_cand
  for (uint32_t i = threadIdx.x; i < n_tiles; i += 256) s_cnt[i] = consume(&a.tile_gt[size_t(row) * a.n_sel_tiles + i]);
  __syncthreads();
  for (uint32_t j = threadIdx.x; j < C; j += 256) {
    const uint64_t c = consume(&clist[j]);
    const uint32_t t = uint32_t(c >> 32);
    if (is_selected(uint32_t(c), int(t), kstar, istar)) atomicAdd(&s_cnt[t / kSelTile], 1u);
  }
  __syncthreads();
  constexpr int PER = kMaxSelTiles / 256;
  uint32_t local = 0;
  for (int j = 0; j < PER; ++j) {
    const uint32_t i = threadIdx.x * PER + j;
    local += (i < n_tiles) ? s_cnt[i] : 0u;
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan(local, s_scan, &total);
  for (int j = 0; j < PER; ++j) {
    const uint32_t i = threadIdx.x * PER + j;
    if (i < n_tiles) {
      a.tile_off[size_t(row) * a.n_sel_tiles + i] = run;
      run += s_cnt[i];
    }
  }
  if (threadIdx.x == 0) {
    g_state[RS_KSTAR] = kstar;
    g_state[RS_ISTAR] = istar;
    g_state[RS_NSCAN] = total;
    publish(&g_state[RS_CAND_COUNT], 0u);
  }
}

__global__ __launch_bounds__(256) void emit_kernel(SelArgs a) {
  __shared__ uint32_t s_wc[4];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int row = b * a.Hkv + h;
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  const int kk = a.topk < n_cand ? a.topk : n_cand;
  const int nW = a.window < Tb ? a.window : Tb;
  int32_t* out = a.idx + size_t(row) * (a.topk + a.window);
  if (tile == 0) {
    for (int j = threadIdx.x; j < nW; j += 256) out[kk + j] = Tb - nW + j;
    if (threadIdx.x == 0) a.n_sel[row] = kk + nW;
  }
  const int t0 = tile * kSelTile;
  if (kk == 0 || t0 >= n_cand) return;
  const int t_end = min(t0 + kSelTile, n_cand);
  if (kk == n_cand) {  // every candidate is selected
    for (int t = t0 + threadIdx.x; t < t_end; t += 256) out[t] = t;
    return;
  }
  const uint32_t* g_state = a.row_state + size_t(row) * kRowStateWords;
  const uint32_t kstar = g_state[RS_KSTAR], istar = g_state[RS_ISTAR];
  const float* srow = a.scores + size_t(row) * a.t_max;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t run = a.tile_off[size_t(row) * a.n_sel_tiles + tile];
  for (int base = t0; base < t_end; base += 256) {
    const int t = base + threadIdx.x;
    bool sel = false;
    if (t < t_end) sel = is_selected(score_key(srow[t]), t, kstar, istar);
    const unsigned long long m = __ballot(sel);
    if (lane == 0) s_wc[wave] = uint32_t(__popcll(m));
    __syncthreads();
    uint32_t woff = 0, tot = 0;
    for (int w = 0; w < 4; ++w) {
      woff += (w < wave) ? s_wc[w] : 0u;
      tot += s_wc[w];
    }
    const uint32_t at = run + woff + uint32_t(__popcll(m & ((1ull << lane) - 1ull)));
    if (sel && at < uint32_t(kk)) out[at] = t;
    run += tot;
    __syncthreads();
  }
}

// ---- launcher -------------------------------------------------------------------------
hipError_t launch_topk(const jssa_desc& d, const float* scores, const int32_t* seq_lens,
                       int32_t* idx, int32_t* n_sel, char* ws_base, const Workspace& ws,
                       bool hist_done, hipStream_t s, hipEvent_t after_select) {
  if (!hist_done) {
    hipError_t e = launch_hist(d, scores, seq_lens, ws_base, ws, s);
    if (e != hipSuccess) return e;
  }
  SelArgs a;
  a.scores = scores; a.seq_lens = seq_lens; a.idx = idx; a.n_sel = n_sel;
  a.row_state = reinterpret_cast<uint32_t*>(ws_base + ws.row_state);
  a.tile_gt = reinterpret_cast<uint32_t*>(ws_base + ws.tile_gt);
  a.tile_off = reinterpret_cast<uint32_t*>(ws_base + ws.tile_off);
  a.cand = reinterpret_cast<uint64_t*>(ws_base + ws.cand);
  a.hist2 = reinterpret_cast<uint32_t*>(ws_base + ws.hist2);
  a.Hkv = d.n_kv_heads; a.t_max = d.t_max; a.topk = d.topk; a.window = d.window;
  a.n_sel_tiles = ws.n_sel_tiles;
  dim3 grid(ws.n_sel_tiles, d.n_kv_heads, d.batch);
  hipLaunchKernelGGL(select_kernel, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (after_select) {
    e = hipEventRecord(after_select, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(emit_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace jssa
