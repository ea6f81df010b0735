// Gather-free indexed attention and the full-KV decode comparison path.
//
// JSSA summary section 3.3: the query heads of a KV head attend over that
// head's own selected positions, reading the selected K/V rows in place from
// the standard [B, T, Hkv, d] cache (no gather buffer), with all KV heads in
// one launch.  Here each workgroup takes one chunk of one (sequence, KV head)
// index list; every K/V row it loads is used by all G query heads of the KV
// head.  Chunks keep an online-softmax state (max, sum, unnormalised output)
// and the last chunk of a row to finish merges them with a log-sum-exp
// combine in a fixed order.  The dense path is the same kernel with the index
// list replaced by 0 .. T_b-1 (JSSA summary section 4.5 compares against
// full-KV decoding).
#include "jssa_device.hpp"
#include "jssa_internal.hpp"

namespace jssa {

constexpr int kMaxIdxChunk = 1024;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  const int32_t* n_sel;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  float* part_acc;
  float* part_ml;
  uint32_t* row_state;
  int Hq, Hkv, t_max, idx_stride, chunk, n_chunks, out_dtype;
  float qscale;  // softmax scale * log2(e): logits are kept in base 2
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int KVT, int D, int G, bool INDEXED>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int EB = Elem<KVT>::bytes;
  constexpr int EPL = Elem<KVT>::per16;
  constexpr int LR = D / EPL;   // lanes per K/V row
  constexpr int RPW = 64 / LR;  // rows per wave per load
  constexpr int NS = 4 * RPW;   // token streams per workgroup
  constexpr int U = 4;          // tokens per stream per step
  static_assert(LR >= 4 && LR <= 32, "row split");

  __shared__ int s_idx[INDEXED ? kMaxIdxChunk : 1];
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_acc[4][G][D];

  const int chunk_id = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int row = b * a.Hkv + h;
  int n;
  if constexpr (INDEXED) {
    n = a.n_sel[row];
    n = n < 0 ? 0 : (n > a.idx_stride ? a.idx_stride : n);
  } else {
    n = a.seq_lens[b];
    n = n < 0 ? 0 : (n > a.t_max ? a.t_max : n);
  }
  const int c0 = chunk_id * a.chunk;
  if (c0 >= n) {
    if (n == 0 && chunk_id == 0) {  // nothing attended: out = 0, lse = -inf
      for (int j = threadIdx.x; j < G * D; j += 256) {
        const size_t o = (size_t(b) * a.Hq + size_t(h) * G) * D + j;
        if (a.out_dtype == JSSA_BF16) reinterpret_cast<uint16_t*>(a.out)[o] = 0;
        else reinterpret_cast<float*>(a.out)[o] = 0.f;
      }
      if (a.lse && threadIdx.x < G) a.lse[size_t(b) * a.Hq + h * G + threadIdx.x] = -INFINITY;
    }
    return;
  }
  const int cnt = min(c0 + a.chunk, n) - c0;
  if constexpr (INDEXED) {
    const int32_t* src = a.idx + size_t(row) * a.idx_stride + c0;
    for (int i = threadIdx.x; i < cnt; i += 256) s_idx[i] = src[i];
    __syncthreads();
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

  for (int i0 = 0; i0 < cnt; i0 += NS * U) {
    uint4 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NS + sidx;
      valid[u] = i < cnt;
      int t = 0;
      if (valid[u]) t = INDEXED ? min(max(s_idx[i], 0), a.t_max - 1) : c0 + i;  // indices are clamped
      const size_t off = head_off + size_t(t) * row_stride;
      if (valid[u]) {
        kr[u] = load16(kbase + off);
        vr[u] = load16(vbase + off);
      } else {
        kr[u] = make_uint4(0u, 0u, 0u, 0u);
        vr[u] = kr[u];
      }
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
      if (lane == 0) { s_m[wave][g] = m[g]; s_l[wave][g] = l[g]; }
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][g][p * EPL + e] = acc[g][e];
    }
  }
  __syncthreads();

  // merge the 4 waves -> this chunk's partial state, published for the combine
  float* pacc = a.part_acc + (size_t(row) * a.n_chunks + chunk_id) * G * D;
  float* pml = a.part_ml + (size_t(row) * a.n_chunks + chunk_id) * G * 2;
  for (int j = threadIdx.x; j < G * D; j += 256) {
    const int g = j / D, dd = j - g * D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = (s_m[w][g] == -INFINITY) ? 0.f : fast_exp2(s_m[w][g] - M);
      L = fmaf(s_l[w][g], sc, L);
      A = fmaf(s_acc[w][g][dd], sc, A);
    }
    publish(&pacc[j], A);
    if (dd == 0) { publish(&pml[2 * g], M); publish(&pml[2 * g + 1], L); }
  }

  // the last chunk of the row combines all chunks in a fixed order
  const uint32_t n_chunks_row = uint32_t((n + a.chunk - 1) / a.chunk);
  uint32_t* ticket = a.row_state + size_t(row) * kRowStateWords + RS_TICKET_ATTN;
  if (!last_arrival(ticket, n_chunks_row)) return;
  const float* racc = a.part_acc + size_t(row) * a.n_chunks * G * D;
  const float* rml = a.part_ml + size_t(row) * a.n_chunks * G * 2;
  constexpr int CB = 8;  // chunks whose loads are issued together
  for (int j = threadIdx.x; j < G * D; j += 256) {
    const int g = j / D, dd = j - g * D;
    float M = -INFINITY;
    for (uint32_t c0 = 0; c0 < n_chunks_row; c0 += CB) {
      float mc[CB];
#pragma unroll
      for (int i = 0; i < CB; ++i)
        mc[i] = (c0 + i < n_chunks_row) ? consume(&rml[((c0 + i) * G + g) * 2]) : -INFINITY;
#pragma unroll
      for (int i = 0; i < CB; ++i) M = fmaxf(M, mc[i]);
    }
    float L = 0.f, A = 0.f;
    for (uint32_t c0 = 0; c0 < n_chunks_row; c0 += CB) {
      float mc[CB], lc[CB], ac[CB];
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const bool ok = c0 + i < n_chunks_row;
        mc[i] = ok ? consume(&rml[((c0 + i) * G + g) * 2]) : -INFINITY;
        lc[i] = ok ? consume(&rml[((c0 + i) * G + g) * 2 + 1]) : 0.f;
        ac[i] = ok ? consume(&racc[(size_t(c0 + i) * G + g) * D + dd]) : 0.f;
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

// ---- launchers ----------------------------------------------------------------------------
template <int KVT, int D, int G>
static hipError_t launch_attn_t(const AttnArgs& args, bool indexed, dim3 grid, hipStream_t s) {
  if (indexed) hipLaunchKernelGGL((attn_kernel<KVT, D, G, true>), grid, dim3(256), 0, s, args);
  else hipLaunchKernelGGL((attn_kernel<KVT, D, G, false>), grid, dim3(256), 0, s, args);
  return hipGetLastError();
}

template <int KVT, int D>
static hipError_t dispatch_g(const AttnArgs& args, int G, bool indexed, dim3 grid, hipStream_t s) {
  switch (G) {
    case 1: return launch_attn_t<KVT, D, 1>(args, indexed, grid, s);
    case 2: return launch_attn_t<KVT, D, 2>(args, indexed, grid, s);
    case 4: return launch_attn_t<KVT, D, 4>(args, indexed, grid, s);
    case 8: return launch_attn_t<KVT, D, 8>(args, indexed, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(const jssa_desc& d, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* idx, const int32_t* n_sel,
                            const int32_t* seq_lens, void* out, float* lse, char* ws_base,
                            const Workspace& ws, hipStream_t s) {
  AttnArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.idx = idx; a.n_sel = n_sel; a.seq_lens = seq_lens;
  a.out = out; a.lse = lse;
  a.part_acc = reinterpret_cast<float*>(ws_base + ws.part_acc);
  a.part_ml = reinterpret_cast<float*>(ws_base + ws.part_ml);
  a.row_state = reinterpret_cast<uint32_t*>(ws_base + ws.row_state);
  a.Hq = d.n_q_heads; a.Hkv = d.n_kv_heads; a.t_max = d.t_max;
  a.idx_stride = d.topk + d.window; a.chunk = ws.chunk; a.n_chunks = ws.n_chunks;
  a.out_dtype = d.out_dtype;
  a.qscale = d.scale * kLog2e;
  const bool indexed = idx != nullptr;
  const int G = d.n_q_heads / d.n_kv_heads;
  dim3 grid(ws.n_chunks, d.n_kv_heads, d.batch);
  if (d.kv_dtype == JSSA_BF16) {
    if (d.d_k == 128) return dispatch_g<1, 128>(a, G, indexed, grid, s);
    if (d.d_k == 64) return dispatch_g<1, 64>(a, G, indexed, grid, s);
  } else {
    if (d.d_k == 128) return dispatch_g<0, 128>(a, G, indexed, grid, s);
    if (d.d_k == 64) return dispatch_g<0, 64>(a, G, indexed, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace jssa
