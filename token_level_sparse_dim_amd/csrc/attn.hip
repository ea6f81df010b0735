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
#include "resolve.hpp"

namespace jssa {

constexpr int kMaxIdxChunk = 1024;
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
    const uint32_t done = __hip_atomic_fetch_add(&a.queue[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == uint32_t(a.n_items) - 1u) {
      __hip_atomic_store(&a.queue[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.queue[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// One chunk of one row: positions [chunk_id*chunk, ...) of the row's n
// tokens; for the indexed path their token indices are already in S.idx.
template <int KVT, int D, int G, bool INDEXED, bool RESOLVE>
__device__ void attend_chunk(const AttnArgs& a, AttnSmem<G, D, INDEXED, RESOLVE>& S, int row, int b,
                             int h, int chunk_id, int n) {
  constexpr int EB = Elem<KVT>::bytes;
  constexpr int EPL = Elem<KVT>::per16;
  constexpr int LR = D / EPL;   // lanes per K/V row
  constexpr int RPW = 64 / LR;  // rows per wave per load
  constexpr int NS = 4 * RPW;   // token streams per workgroup
  constexpr int U = JSSA_ATTN_UNROLL;  // tokens per stream per step
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
  if (!last_arrival(&rstate[RS_TICKET_ATTN], uint32_t(a.n_chunks))) return;
  if (RESOLVE && threadIdx.x == 0) publish(&rstate[RS_READY], 0u);  // every chunk has passed its wait
  const uint32_t n_live = uint32_t((n + a.chunk - 1) / a.chunk);
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
  constexpr int CB = 8;  // chunks whose loads are issued together
  for (int j = threadIdx.x; j < G * D; j += 256) {
    const int g = j / D, dd = j - g * D;
    float M = -INFINITY;
    for (uint32_t cb = 0; cb < n_live; cb += CB) {
      float mc[CB];
#pragma unroll
      for (int i = 0; i < CB; ++i)
        mc[i] = (cb + i < n_live) ? consume(&rml[((cb + i) * G + g) * 2]) : -INFINITY;
#pragma unroll
      for (int i = 0; i < CB; ++i) M = fmaxf(M, mc[i]);
    }
    float L = 0.f, A = 0.f;
    for (uint32_t cb = 0; cb < n_live; cb += CB) {
      float mc[CB], lc[CB], ac[CB];
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const bool ok = cb + i < n_live;
        mc[i] = ok ? consume(&rml[((cb + i) * G + g) * 2]) : -INFINITY;
        lc[i] = ok ? consume(&rml[((cb + i) * G + g) * 2 + 1]) : 0.f;
        ac[i] = ok ? consume(&racc[(size_t(cb + i) * G + g) * D + dd]) : 0.f;
      }
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const float w = (mc[i] == -INFINITY) ? 0.f : fast_exp2(mc[i] - M);
        L = fmaf(lc[i], w, L);
        A = fmaf(ac[i], w, A);
      }
    }
    const float o = A / L;
    const size_t oi = (size_t(b) * a.Hq + size_t(h) * G + g) * D + dd;
    if (a.out_dtype == JSSA_BF16) reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(o);
    else reinterpret_cast<float*>(a.out)[oi] = o;
    if (dd == 0 && a.lse) a.lse[size_t(b) * a.Hq + h * G + g] = (M + __log2f(L)) * kLn2;
  }
}

template <int KVT, int D, int G, bool INDEXED, bool RESOLVE>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  using ASmem = AttnSmem<G, D, INDEXED, RESOLVE>;
  constexpr size_t kSmem = (RESOLVE && sizeof(ResolveSmem) > sizeof(ASmem)) ? sizeof(ResolveSmem) : sizeof(ASmem);
  __shared__ __align__(16) char smem_raw[kSmem];
  __shared__ uint32_t s_item;

  if (threadIdx.x == 0) s_item = __hip_atomic_fetch_add(&a.queue[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      if (spins >= kSpinLimit) publish(&a.queue[2], 1u);  // broken invariant: flagged, not hung
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
