// Exact resolution of one (sequence, KV head) selection (JSSA summary
// Figure 1 and section 3.1: each KV head keeps its own top-k positions; ties
// go to the lower index), and the extraction of any range of the resulting
// ascending index list.
//
// Inputs: the first-digit threshold bin D1 with the number of keys still
// needed from it (from the histogram of the score scan), and the candidates
// of every selection tile -- all keys whose top 12 bits are >= D1, i.e. every
// token that can be selected -- stored in token order in per-tile slots by the
// candidate pass (select.hip).
//
// resolve_row (one workgroup per row) finds the exact k-th key K* and the tie
// cut I* from the candidates in bin D1, and publishes, per tile, where the
// tile's selected tokens start in the output list (tile_off) and where its
// candidates start in the concatenated candidate list (cand_base).
// extract_range (any workgroup) then rebuilds positions [p0, p1) of the index
// list from those tables, so the emission is spread over the attention items.
#pragma once

#include "jssa_device.hpp"
#include "jssa_internal.hpp"
#include "select_common.hpp"

namespace jssa {

constexpr int kBinLds = 4096;  // bin-D1 candidates resolved in shared memory

struct ResolveSmem {
  uint64_t bin[kBinLds];        // candidates in bin D1 (any order)
  uint32_t tab[kMaxSelTiles];   // candidate prefix, then per-tile selected counts
  uint32_t hist[1024];
  uint32_t scan[8];
  uint32_t out[2];
  uint32_t n_bin;
};

struct ResolveArgs {
  const int32_t* seq_lens;
  const uint32_t* tile_cnt;  // [rows][n_sel_tiles] candidates per tile (previous launch)
  const uint64_t* cand;      // [rows][t_max] tile slots (previous launch)
  uint32_t* row_state;
  uint32_t* tile_off;        // [rows][n_sel_tiles] published here
  uint32_t* cand_base;       // [rows][n_sel_tiles] published here
  int32_t* n_sel;            // [rows]
  int t_max, topk, window, n_sel_tiles;
};

__device__ __forceinline__ bool passes(uint64_t c, uint32_t kstar, uint32_t istar) {
  const uint32_t key = uint32_t(c), t = uint32_t(c >> 32);
  return key > kstar || (key == kstar && t <= istar);
}

// Index of the last entry of an ascending table with tab[i] <= v (tab[0] <= v).
__device__ __forceinline__ uint32_t last_le(const uint32_t* tab, uint32_t n, uint32_t v) {
  uint32_t lo = 0, hi = n;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (tab[mid] <= v) lo = mid; else hi = mid;
  }
  return lo;
}

// K* and I* from the candidates in bin D1 (read through `get`, n of them).
template <typename Get>
__device__ void cut_from_bin(Get get, uint32_t n, uint32_t D1, uint32_t need1, ResolveSmem& sm,
                             uint32_t* kstar_out, uint32_t* istar_out) {
  // digit 2: key bits 19..10
  for (int i = threadIdx.x; i < 1024; i += 256) sm.hist[i] = 0u;
  __syncthreads();
  for (uint32_t j = threadIdx.x; j < n; j += 256) {
    const uint32_t key = uint32_t(get(j));
    if ((key >> (32 - kDigit1Bits)) == D1) atomicAdd(&sm.hist[(key >> 10) & 0x3ffu], 1u);
  }
  __syncthreads();
  find_bin_from_top<4>(sm.hist, need1, sm.scan, sm.out);
  const uint32_t D2 = sm.out[0];
  const uint32_t need2 = need1 - sm.out[1];
  __syncthreads();
  const uint32_t hi22 = (D1 << 10) | D2;
  // digit 3: key bits 9..0
  for (int i = threadIdx.x; i < 1024; i += 256) sm.hist[i] = 0u;
  __syncthreads();
  for (uint32_t j = threadIdx.x; j < n; j += 256) {
    const uint32_t key = uint32_t(get(j));
    if ((key >> 10) == hi22) atomicAdd(&sm.hist[key & 0x3ffu], 1u);
  }
  __syncthreads();
  find_bin_from_top<4>(sm.hist, need2, sm.scan, sm.out);
  const uint32_t D3 = sm.out[0];
  const uint32_t m_ties = need2 - sm.out[1];  // keys equal to K* still to take, lowest indices first
  const uint32_t n_eq = sm.hist[D3];
  const uint32_t kstar = (hi22 << 10) | D3;
  __syncthreads();
  uint32_t istar = 0xffffffffu;
  if (m_ties < n_eq) {
    // the m_ties-th smallest index among keys equal to K*: index bits 23..16, 15..8, 7..0
    uint32_t prefix = 0, m = m_ties;
    for (int shift = 16; shift >= 0; shift -= 8) {
      if (threadIdx.x < 256) sm.hist[threadIdx.x] = 0u;
      __syncthreads();
      for (uint32_t j = threadIdx.x; j < n; j += 256) {
        const uint64_t c = get(j);
        const uint32_t t = uint32_t(c >> 32);
        if (uint32_t(c) == kstar && (t >> (shift + 8)) == (prefix >> (shift + 8)))
          atomicAdd(&sm.hist[(t >> shift) & 0xffu], 1u);
      }
      __syncthreads();
      find_bin_from_bottom<1>(sm.hist, m, sm.scan, sm.out);
      prefix |= sm.out[0] << shift;
      m -= sm.out[1];
      __syncthreads();
    }
    istar = prefix;
  }
  *kstar_out = kstar;
  *istar_out = istar;
}

// One workgroup per row.  Publishes n_sel[row], and for rows that need a cut
// RS_KSTAR / RS_ISTAR and the tile_off / cand_base tables.
__device__ void resolve_row(const ResolveArgs& a, int b, int row, ResolveSmem& sm) {
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  const int kk = a.topk < n_cand ? a.topk : n_cand;
  const int nW = a.window < Tb ? a.window : Tb;
  if (threadIdx.x == 0) publish(reinterpret_cast<uint32_t*>(a.n_sel + row), uint32_t(kk + nW));
  if (kk == 0 || kk == n_cand) return;  // nothing to cut
  uint32_t* g_state = a.row_state + size_t(row) * kRowStateWords;
  const uint32_t D1 = g_state[RS_D1], need1 = g_state[RS_NEED1];
  const uint32_t n_tiles = uint32_t((n_cand + kSelTile - 1) / kSelTile);
  const uint32_t* cnt = a.tile_cnt + size_t(row) * a.n_sel_tiles;
  const uint64_t* slots = a.cand + size_t(row) * a.t_max;
  constexpr int PER = kMaxSelTiles / 256;

  // exclusive prefix of candidate counts -> sm.tab and cand_base
  uint32_t c[PER], local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t i = threadIdx.x * PER + j;
    c[j] = (i < n_tiles) ? cnt[i] : 0u;
    local += c[j];
  }
  uint32_t C;
  uint32_t run = block_exclusive_scan(local, sm.scan, &C);
  uint32_t* g_base = a.cand_base + size_t(row) * a.n_sel_tiles;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t i = threadIdx.x * PER + j;
    sm.tab[i] = run;
    if (i < n_tiles) publish(&g_base[i], run);
    run += c[j];
  }
  if (threadIdx.x == 0) sm.n_bin = 0u;
  __syncthreads();

  // gather the candidates of bin D1 (loads issued in batches)
  constexpr int BATCH = 8;
  for (uint32_t j0 = 0; j0 < C; j0 += 256 * BATCH) {
    uint64_t v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const uint32_t j = min(j0 + u * 256 + threadIdx.x, C - 1);
      const uint32_t tile = last_le(sm.tab, n_tiles, j);
      v[u] = slots[size_t(tile) * kSelTile + (j - sm.tab[tile])];
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const uint32_t j = j0 + u * 256 + threadIdx.x;
      if (j < C && (uint32_t(v[u]) >> (32 - kDigit1Bits)) == D1) {
        const uint32_t at = atomicAdd(&sm.n_bin, 1u);
        if (at < uint32_t(kBinLds)) sm.bin[at] = v[u];
      }
    }
  }
  __syncthreads();
  const uint32_t n_bin = sm.n_bin;
  const bool bin_in_lds = n_bin <= uint32_t(kBinLds);
  // the j-th candidate of the row (any bin), addressed through the prefix in sm.tab
  auto cand_at = [&](uint32_t j) {
    const uint32_t tile = last_le(sm.tab, n_tiles, j);
    return slots[size_t(tile) * kSelTile + (j - sm.tab[tile])];
  };
  uint32_t kstar, istar;
  if (bin_in_lds) {
    cut_from_bin([&](uint32_t j) { return sm.bin[j]; }, n_bin, D1, need1, sm, &kstar, &istar);
  } else {
    // more bin-D1 candidates than fit: read every candidate; the digit tests of
    // the cut only count keys in bin D1
    cut_from_bin(cand_at, C, D1, need1, sm, &kstar, &istar);
  }

  // per-tile selected counts: every candidate above bin D1 passes; bin-D1 ones by the cut
  uint32_t* selc = bin_in_lds ? sm.tab : reinterpret_cast<uint32_t*>(sm.bin);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) selc[threadIdx.x * PER + j] = c[j];
  __syncthreads();
  if (bin_in_lds) {
    for (uint32_t j = threadIdx.x; j < n_bin; j += 256) {
      const uint64_t v = sm.bin[j];
      if (!passes(v, kstar, istar)) atomicSub(&selc[uint32_t(v >> 32) / kSelTile], 1u);
    }
  } else {
    for (uint32_t j = threadIdx.x; j < C; j += 256) {
      const uint64_t v = cand_at(j);
      if ((uint32_t(v) >> (32 - kDigit1Bits)) == D1 && !passes(v, kstar, istar))
        atomicSub(&selc[uint32_t(v >> 32) / kSelTile], 1u);
    }
  }
  __syncthreads();
  uint32_t sel[PER], loc = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    sel[j] = selc[threadIdx.x * PER + j];
    loc += sel[j];
  }
  uint32_t total;
  uint32_t pos = block_exclusive_scan(loc, sm.scan, &total);
  uint32_t* g_off = a.tile_off + size_t(row) * a.n_sel_tiles;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t i = threadIdx.x * PER + j;
    if (i < n_tiles) publish(&g_off[i], pos);
    pos += sel[j];
  }
  if (threadIdx.x == 0) {
    publish(&g_state[RS_KSTAR], kstar);
    publish(&g_state[RS_ISTAR], istar);
    publish(&g_state[RS_NCAND], C);
  }
}

// Positions [p0, p1) of the row's index list into dst[0 .. p1-p0), and into
// idx_out (when given) at the same positions.  After the row's resolve has
// been published.  Every thread of the workgroup calls it; `tab` holds
// 2*kMaxSelTiles words of shared memory and `scan` 8 words.
__device__ void extract_range(const ResolveArgs& a, int b, int row, int p0, int p1, int* dst,
                              int32_t* idx_out, uint32_t* tab, uint32_t* scan) {
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  const int kk = a.topk < n_cand ? a.topk : n_cand;
  const int nW = a.window < Tb ? a.window : Tb;
  // the window and the "every candidate" case are arithmetic
  for (int p = p0 + threadIdx.x; p < p1; p += 256) {
    int t = -1;
    if (p >= kk) t = Tb - nW + (p - kk);
    else if (kk == n_cand) t = p;
    if (t >= 0) {
      dst[p - p0] = t;
      if (idx_out) idx_out[p] = t;
    }
  }
  const int q1 = min(p1, kk);
  if (kk == n_cand || p0 >= q1) {
    __syncthreads();
    return;
  }
  // selected positions [p0, q1): from the tiles whose output ranges overlap it
  const uint32_t* g_state = a.row_state + size_t(row) * kRowStateWords;
  const uint32_t kstar = consume(&g_state[RS_KSTAR]), istar = consume(&g_state[RS_ISTAR]);
  const uint32_t C = consume(&g_state[RS_NCAND]);
  const uint32_t n_tiles = uint32_t((n_cand + kSelTile - 1) / kSelTile);
  uint32_t* toff = tab;
  uint32_t* cbase = tab + kMaxSelTiles;
  const uint32_t* g_off = a.tile_off + size_t(row) * a.n_sel_tiles;
  const uint32_t* g_base = a.cand_base + size_t(row) * a.n_sel_tiles;
  for (uint32_t i = threadIdx.x; i < n_tiles; i += 256) {
    toff[i] = consume(&g_off[i]);
    cbase[i] = consume(&g_base[i]);
  }
  __syncthreads();
  const uint32_t first = last_le(toff, n_tiles, uint32_t(p0));
  const uint32_t last = last_le(toff, n_tiles, uint32_t(q1 - 1));
  const uint32_t j_begin = cbase[first];
  const uint32_t j_end = (last + 1 < n_tiles) ? cbase[last + 1] : C;
  const uint64_t* slots = a.cand + size_t(row) * a.t_max;
  // ordered compaction of the passing candidates in [j_begin, j_end), 256 at a time
  uint32_t run = toff[first];  // output position of the first passing candidate of `first`
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (uint32_t j0 = j_begin; j0 < j_end && run < uint32_t(q1); j0 += 256) {
    const uint32_t j = j0 + threadIdx.x;
    bool ok = false;
    uint32_t t = 0;
    if (j < j_end) {
      const uint32_t tile = last_le(cbase, n_tiles, j);
      const uint64_t v = slots[size_t(tile) * kSelTile + (j - cbase[tile])];
      ok = passes(v, kstar, istar);
      t = uint32_t(v >> 32);
    }
    const unsigned long long bal = __ballot(ok);
    if (lane == 0) scan[wave] = uint32_t(__popcll(bal));
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t cw = scan[w];
      before += (w < wave) ? cw : 0u;
      tot += cw;
    }
    if (ok) {
      const uint32_t p = run + before + uint32_t(__popcll(bal & ((1ull << lane) - 1ull)));
      if (p >= uint32_t(p0) && p < uint32_t(q1)) {
        dst[p - p0] = int(t);
        if (idx_out) idx_out[p] = int(t);
      }
    }
    run += tot;
    __syncthreads();
  }
  __syncthreads();
}

}  // namespace jssa
