// Gather-free indexed attention and the full-KV decode comparison path.
//
// JSSA summary section 3.3: the query heads of a KV head attend over that
// head's own selected positions, reading the selected K/V rows in place from
// the standard [B, T, Hkv, d] cache (no gather buffer), with all KV heads in
// one launch.  Here each attention item is one chunk of one (sequence, KV
// head) index list; every K/V row it loads is used by all G query heads of
// the KV head.  Chunks keep an online-softmax state (max, sum, unnormalised
// output) and the last chunk of a row to finish merges them with a
// log-sum-exp combine in a fixed order.  The dense path is the same code with
// the index list replaced by 0 .. T_b-1 (JSSA summary section 4.5 compares
// against full-KV decoding).
//
// The resolve items of the selection (resolve.hpp) run in the same launch:
// workgroups take items from a queue in order, resolve items first, and an
// attention chunk waits until its row's selection is published.  A waiting
// chunk only waits for items handed out before it, whose workgroups are
// already running, so the wait always ends; rows whose selection is done are
// attended while other rows are still resolving.
#include "jssa_device.hpp"
#include "jssa_internal.hpp"
#include "attn_core.hpp"
#include "resolve.hpp"

namespace jssa {

template <int KVT, int D, int G, bool INDEXED, bool RESOLVE>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  using ASmem = AttnSmem<G, D, INDEXED, RESOLVE>;
  constexpr size_t kSmem = (RESOLVE && sizeof(ResolveSmem) > sizeof(ASmem)) ? sizeof(ResolveSmem) : sizeof(ASmem);
  __shared__ __align__(16) char smem_raw[kSmem];
  __shared__ uint32_t s_item;

  if (threadIdx.x == 0) s_item = __hip_atomic_fetch_add(&a.queue[QW_NEXT], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int item = int(s_item);
  if (RESOLVE && item < a.n_resolve) {
    const int row = item, b = row / a.Hkv;
    resolve_row(a.res, b, row, *reinterpret_cast<ResolveSmem*>(smem_raw));
    __builtin_amdgcn_s_waitcnt(0);  // the row's tables are published before it is marked ready
    __syncthreads();
    if (threadIdx.x == 0) publish(&a.row_state[size_t(row) * kRowStateWords + RS_READY], 1u);
    finish_item(a);
    return;
  }
  ASmem& S = *reinterpret_cast<ASmem*>(smem_raw);
  const int it = item - a.n_resolve;
  const int row = it / a.n_chunks, chunk_id = it - row * a.n_chunks;
  const int b = row / a.Hkv, h = row - b * a.Hkv;
  uint32_t* rstate = a.row_state + size_t(row) * kRowStateWords;
  if (RESOLVE) {  // wait until this row's selection is published
    if (threadIdx.x == 0) {
      uint32_t spins = 0;
      while (consume(&rstate[RS_READY]) == 0u && ++spins < kSpinLimit) __builtin_amdgcn_s_sleep(2);
      if (spins >= kSpinLimit) publish(&a.queue[QW_ERR], 1u);  // broken invariant: flagged, not hung
    }
    __syncthreads();
  }
  int n;
  if constexpr (INDEXED) {
    n = int(consume(reinterpret_cast<const uint32_t*>(a.n_sel + row)));
    n = n < 0 ? 0 : (n > a.idx_stride ? a.idx_stride : n);
  } else {
    n = a.seq_lens[b];
    n = n < 0 ? 0 : (n > a.t_max ? a.t_max : n);
  }
  if constexpr (INDEXED) {  // this chunk's token indices -> S.idx
    const int c0 = chunk_id * a.chunk;
    const int cnt = c0 < n ? min(c0 + a.chunk, n) - c0 : 0;
    if (cnt > 0) {
      if constexpr (RESOLVE) {
        extract_range(a.res, b, row, c0, c0 + cnt, S.idx, a.idx + size_t(row) * a.idx_stride, S.tab, S.scan);
      } else {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.idx + size_t(row) * a.idx_stride + c0);
        for (int i = threadIdx.x; i < cnt; i += 256) S.idx[i] = int(consume(&src[i]));
        __syncthreads();
      }
    }
  }
  if (a.attend) {
    attend_chunk<KVT, D, G, INDEXED, RESOLVE>(a, S, row, b, h, chunk_id, n);
  } else if (last_arrival(&rstate[RS_TICKET_ATTN], uint32_t(a.n_chunks))) {
    if (RESOLVE && threadIdx.x == 0) publish(&rstate[RS_READY], 0u);  // every chunk has passed its wait
  }
  finish_item(a);
}

// ---- launchers ----------------------------------------------------------------------------
template <int KVT, int D, int G>
static hipError_t launch_attn_t(const AttnArgs& args, bool indexed, bool resolve, dim3 grid, hipStream_t s) {
  if (resolve) hipLaunchKernelGGL((attn_kernel<KVT, D, G, true, true>), grid, dim3(256), 0, s, args);
  else if (indexed) hipLaunchKernelGGL((attn_kernel<KVT, D, G, true, false>), grid, dim3(256), 0, s, args);
  else hipLaunchKernelGGL((attn_kernel<KVT, D, G, false, false>), grid, dim3(256), 0, s, args);
  return hipGetLastError();
}

template <int KVT, int D>
static hipError_t dispatch_g(const AttnArgs& args, int G, bool indexed, bool resolve, dim3 grid, hipStream_t s) {
  switch (G) {
    case 1: return launch_attn_t<KVT, D, 1>(args, indexed, resolve, grid, s);
    case 2: return launch_attn_t<KVT, D, 2>(args, indexed, resolve, grid, s);
    case 4: return launch_attn_t<KVT, D, 4>(args, indexed, resolve, grid, s);
    case 8: return launch_attn_t<KVT, D, 8>(args, indexed, resolve, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_resolve_attend(const jssa_desc& d, bool resolve, bool attend, const void* q,
                                 const void* k_cache, const void* v_cache, int32_t* idx,
                                 int32_t* n_sel, const int32_t* seq_lens, void* out, float* lse,
                                 char* ws_base, const Workspace& ws, hipStream_t s) {
  AttnArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.idx = idx; a.n_sel = n_sel; a.seq_lens = seq_lens;
  a.attend = attend ? 1 : 0;
  a.out = out; a.lse = lse;
  a.part_acc = reinterpret_cast<float*>(ws_base + ws.part_acc);
  a.part_ml = reinterpret_cast<float*>(ws_base + ws.part_ml);
  a.row_state = reinterpret_cast<uint32_t*>(ws_base + ws.row_state);
  a.queue = reinterpret_cast<uint32_t*>(ws_base + ws.queue);
  a.Hq = d.n_q_heads; a.Hkv = d.n_kv_heads; a.t_max = d.t_max;
  a.idx_stride = d.topk + d.window;
  if (attend) {
    a.chunk = ws.chunk;
    a.n_chunks = ws.n_chunks;
  } else {  // emission only: the index list in chunks of kMaxIdxChunk
    a.chunk = kMaxIdxChunk;
    a.n_chunks = (a.idx_stride + kMaxIdxChunk - 1) / kMaxIdxChunk;
  }
  a.out_dtype = d.out_dtype;
  a.qscale = d.scale * kLog2e;
  const int rows = d.batch * d.n_kv_heads;
  a.n_resolve = resolve ? rows : 0;
  a.n_items = a.n_resolve + ((attend || resolve) ? rows * a.n_chunks : 0);
  a.res.seq_lens = seq_lens;
  a.res.tile_cnt = reinterpret_cast<const uint32_t*>(ws_base + ws.tile_cnt);
  a.res.cand = reinterpret_cast<const uint64_t*>(ws_base + ws.cand);
  a.res.row_state = a.row_state;
  a.res.tile_off = reinterpret_cast<uint32_t*>(ws_base + ws.tile_off);
  a.res.cand_base = reinterpret_cast<uint32_t*>(ws_base + ws.cand_base);
  a.res.n_sel = n_sel;
  a.res.t_max = d.t_max; a.res.topk = d.topk; a.res.window = d.window;
  a.res.n_sel_tiles = ws.n_sel_tiles;
  if (a.n_items == 0) return hipSuccess;
  const bool indexed = idx != nullptr;
  const int G = d.n_q_heads / d.n_kv_heads;
  dim3 grid(a.n_items);
  if (!attend && !resolve) return hipSuccess;
  if (!attend) return launch_attn_t<1, 128, 1>(a, indexed, resolve, grid, s);  // emission only: no K/V access
  if (d.kv_dtype == JSSA_BF16) {
    if (d.d_k == 128) return dispatch_g<1, 128>(a, G, indexed, resolve, grid, s);
    if (d.d_k == 64) return dispatch_g<1, 64>(a, G, indexed, resolve, grid, s);
  } else {
    if (d.d_k == 128) return dispatch_g<0, 128>(a, G, indexed, resolve, grid, s);
    if (d.d_k == 64) return dispatch_g<0, 64>(a, G, indexed, resolve, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace jssa
