// Candidate pass of the per-(sequence, KV head) top-k (JSSA summary Figure 1
// and section 3.1).  After the score scan has fixed the first-digit threshold
// bin D1 of each row, every workgroup takes one tile of kSelTile scores and
// writes the keys whose top 12 bits are >= D1 -- every token that can be
// selected -- in token order into the tile's slot, with the slot's count.
// The exact cut is made by the resolve items (resolve.hpp), or, with SUB = 4
// (the MLA decode), by the fused decode's selection, which reads the same
// slots per 1024-token sub-tile (counts in `tile_cnt` per sub-tile).
#include "jssa_device.hpp"
#include "jssa_internal.hpp"
#include "select_common.hpp"

namespace jssa {

struct CandArgs {
  const float* scores;
  const int32_t* seq_lens;
  const uint32_t* row_state;
  uint32_t* tile_cnt;
  uint64_t* cand;
  int Hkv, t_max, topk, window, n_sel_tiles;
};

template <int SUB>
__global__ __launch_bounds__(256) void cand_kernel(CandArgs a) {
  constexpr int PER_SUB = kKeysPerThread / SUB;  // key rounds of 256 tokens per sub-tile
  static_assert(PER_SUB * SUB == kKeysPerThread, "sub-tiles of whole rounds");
  __shared__ uint32_t s_wc[4][kKeysPerThread];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int row = b * a.Hkv + h;
  int Tb;
  const int n_cand = candidates_of(a.seq_lens, b, a.t_max, a.window, &Tb);
  if (a.topk <= 0 || a.topk >= n_cand) return;  // nothing to cut: resolved without candidates
  const int t0 = tile * kSelTile;
  if (t0 >= n_cand) return;
  const int t_end = min(t0 + kSelTile, n_cand);
  const uint32_t D1 = a.row_state[size_t(row) * kRowStateWords + RS_D1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t key[kKeysPerThread];
  load_tile_keys(a.scores + size_t(row) * a.t_max, t0, t_end, key);
  unsigned long long bal[kKeysPerThread];
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const int t = t0 + i * 256 + int(threadIdx.x);
    bal[i] = __ballot(t < t_end && (key[i] >> (32 - kDigit1Bits)) >= D1);
    if (lane == 0) s_wc[wave][i] = uint32_t(__popcll(bal[i]));
  }
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub) {
    const int s0 = t0 + sub * PER_SUB * 256;  // the sub-tile's first token
    if (s0 >= t_end) break;
    uint64_t* slot = a.cand + size_t(row) * a.t_max + s0;
    uint32_t run = 0;
#pragma unroll
    for (int i = sub * PER_SUB; i < (sub + 1) * PER_SUB; ++i) {
      uint32_t before = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t c = s_wc[w][i];
        before += (w < wave) ? c : 0u;
        tot += c;
      }
      if ((bal[i] >> lane) & 1ull) {
        const uint32_t t = uint32_t(t0 + i * 256 + int(threadIdx.x));
        publish(&slot[run + before + uint32_t(__popcll(bal[i] & below))], (uint64_t(t) << 32) | key[i]);
      }
      run += tot;
    }
    if (threadIdx.x == 0) publish(&a.tile_cnt[size_t(row) * a.n_sel_tiles * SUB + tile * SUB + sub], run);
  }
}

hipError_t launch_candidates(const jssa_desc& d, const float* scores, const int32_t* seq_lens,
                             char* ws_base, const Workspace& ws, hipStream_t s, bool sub_tiles) {
  CandArgs a;
  a.scores = scores; a.seq_lens = seq_lens;
  a.row_state = reinterpret_cast<const uint32_t*>(ws_base + ws.row_state);
  a.tile_cnt = reinterpret_cast<uint32_t*>(ws_base + ws.tile_cnt);
  a.cand = reinterpret_cast<uint64_t*>(ws_base + ws.cand);
  a.Hkv = d.n_kv_heads; a.t_max = d.t_max; a.topk = d.topk; a.window = d.window;
  a.n_sel_tiles = ws.n_sel_tiles;
  dim3 grid(ws.n_sel_tiles, d.n_kv_heads, d.batch);
  if (sub_tiles) hipLaunchKernelGGL(cand_kernel<kSelTile / kSubTile>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(cand_kernel<1>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace jssa
