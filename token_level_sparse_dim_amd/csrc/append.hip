// Append new K/V rows and project keys into the scoring cache (JSSA summary
// section E.1: each newly generated key is projected; sections 3.1 and 3.4:
// the scoring-only cache holds Kp = K P per KV head).  One lane per token:
// the lane walks its key row in 16-byte pieces and accumulates the rank-R
// projection in fp32; the basis rows are wave-uniform, so they come through
// the scalar cache.
#include "append_core.hpp"
#include "jssa_device.hpp"
#include "jssa_internal.hpp"

namespace jssa {

constexpr int kAppendRowsMax = 64;  // up to this many new rows: one workgroup per row

template <int KVT, int KPT, int R>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int EB = Elem<KVT>::bytes;
  constexpr int EPL = Elem<KVT>::per16;
  const int h = blockIdx.y, b = blockIdx.z;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.n_new) return;
  const int t = a.pos[b] + j;
  if (t < 0 || t >= a.t_max) return;

  char* kc = reinterpret_cast<char*>(a.k_cache);
  const size_t crow = ((size_t(b) * a.t_max + t) * a.Hkv + h) * a.d_k * EB;
  const char* src;
  if (a.k_new) {
    const char* kn = reinterpret_cast<const char*>(a.k_new);
    src = kn + ((size_t(b) * a.n_new + j) * a.Hkv + h) * a.d_k * EB;
    for (int o = 0; o < a.d_k * EB; o += 16) *reinterpret_cast<uint4*>(kc + crow + o) = load16(src + o);
    if (!a.mla && a.v_new) {
      const char* vn = reinterpret_cast<const char*>(a.v_new);
      const char* vs = vn + ((size_t(b) * a.n_new + j) * a.Hkv + h) * a.d_v * EB;
      char* vc = reinterpret_cast<char*>(a.v_cache) + ((size_t(b) * a.t_max + t) * a.Hkv + h) * a.d_v * EB;
      for (int o = 0; o < a.d_v * EB; o += 16) *reinterpret_cast<uint4*>(vc + o) = load16(vs + o);
    }
  } else {
    src = kc + crow;
  }

  float acc[R];
#pragma unroll
  for (int i = 0; i < R; ++i) acc[i] = 0.f;
  const float* Ph = a.P + size_t(h) * a.d_k * R;
  for (int d0 = 0; d0 < a.d_k; d0 += EPL) {
    float kv[EPL];
    unpack16<KVT>(load16(src + size_t(d0) * EB), kv);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float* Pr = Ph + size_t(d0 + e) * R;
#pragma unroll
      for (int i = 0; i < R; ++i) acc[i] = fmaf(kv[e], Pr[i], acc[i]);
    }
  }

  char* kprow = reinterpret_cast<char*>(a.kp) + ((size_t(b) * a.Hkv + h) * a.t_max + t) * R * Elem<KPT>::bytes;
  if constexpr (KPT == 1) {
#pragma unroll
    for (int i = 0; i < R; i += 8) {
      uint4 w;
      w.x = uint32_t(f32_to_bf16_rne(acc[i + 0])) | (uint32_t(f32_to_bf16_rne(acc[i + 1])) << 16);
      w.y = uint32_t(f32_to_bf16_rne(acc[i + 2])) | (uint32_t(f32_to_bf16_rne(acc[i + 3])) << 16);
      w.z = uint32_t(f32_to_bf16_rne(acc[i + 4])) | (uint32_t(f32_to_bf16_rne(acc[i + 5])) << 16);
      w.w = uint32_t(f32_to_bf16_rne(acc[i + 6])) | (uint32_t(f32_to_bf16_rne(acc[i + 7])) << 16);
      *reinterpret_cast<uint4*>(kprow + i * 2) = w;
    }
  } else if constexpr (KPT == 2) {
#pragma unroll
    for (int i = 0; i < R; i += 16) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = f32_to_e4m3_sat(acc[i + 4 * k]) | (f32_to_e4m3_sat(acc[i + 4 * k + 1]) << 8) |
               (f32_to_e4m3_sat(acc[i + 4 * k + 2]) << 16) | (f32_to_e4m3_sat(acc[i + 4 * k + 3]) << 24);
      *reinterpret_cast<uint4*>(kprow + i) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < R; i += 4)
      *reinterpret_cast<float4*>(kprow + i * 4) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
  }
}

// Few new rows (a decode step): one workgroup per (b, j, h) row; the rank-R
// projection is split over 256 threads (R outputs x 256/R slices of d) with
// the basis read coalesced and the key row staged in shared memory.
template <int KVT, int KPT, int R>
__global__ __launch_bounds__(256) void append_rows_kernel(AppendArgs a) {
  constexpr int EB = Elem<KVT>::bytes;
  constexpr int EPL = Elem<KVT>::per16;
  constexpr int PARTS = 256 / R;
  __shared__ float s_k[576];
  __shared__ float s_part[256];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b] + j;
  if (t < 0 || t >= a.t_max) return;
  char* kc = reinterpret_cast<char*>(a.k_cache);
  const size_t crow = ((size_t(b) * a.t_max + t) * a.Hkv + h) * a.d_k * EB;
  const char* src = kc + crow;
  if (a.k_new) src = reinterpret_cast<const char*>(a.k_new) + ((size_t(b) * a.n_new + j) * a.Hkv + h) * a.d_k * EB;
  const int n16 = a.d_k * EB / 16;
  for (int c = threadIdx.x; c < n16; c += 256) {
    const uint4 v = load16(src + size_t(c) * 16);
    float f[EPL];
    unpack16<KVT>(v, f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_k[c * EPL + e] = f[e];
    if (a.k_new) *reinterpret_cast<uint4*>(kc + crow + size_t(c) * 16) = v;
  }
  if (a.k_new && !a.mla && a.v_new) {
    const char* vs = reinterpret_cast<const char*>(a.v_new) + ((size_t(b) * a.n_new + j) * a.Hkv + h) * a.d_v * EB;
    char* vc = reinterpret_cast<char*>(a.v_cache) + ((size_t(b) * a.t_max + t) * a.Hkv + h) * a.d_v * EB;
    for (int c = threadIdx.x; c < a.d_v * EB / 16; c += 256)
      *reinterpret_cast<uint4*>(vc + size_t(c) * 16) = load16(vs + size_t(c) * 16);
  }
  __syncthreads();
  const int o = threadIdx.x % R, part = threadIdx.x / R;
  const int dper = (a.d_k + PARTS - 1) / PARTS;
  const int d0 = part * dper, d1 = min(a.d_k, d0 + dper);
  const float* Pc = a.P + size_t(h) * a.d_k * R + o;
  float acc = 0.f;
#pragma unroll 8
  for (int d = d0; d < d1; ++d) acc = fmaf(s_k[d], Pc[size_t(d) * R], acc);
  s_part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < R) {
    float sum = 0.f;
    for (int pp = 0; pp < PARTS; ++pp) sum += s_part[pp * R + threadIdx.x];
    char* kprow = reinterpret_cast<char*>(a.kp) + ((size_t(b) * a.Hkv + h) * a.t_max + t) * R * Elem<KPT>::bytes;
    if constexpr (KPT == 1) reinterpret_cast<uint16_t*>(kprow)[threadIdx.x] = f32_to_bf16_rne(sum);
    else if constexpr (KPT == 2) reinterpret_cast<uint8_t*>(kprow)[threadIdx.x] = uint8_t(f32_to_e4m3_sat(sum));
    else reinterpret_cast<float*>(kprow)[threadIdx.x] = sum;
  }
}

// The decode step's append (given new rows, d_k = DPER * 256 / R): thread
// (o, part) needs key elements [part*DPER, (part+1)*DPER) and the same rows of
// basis column o; those, the position and the rows to copy into the caches
// are all requested at once, so the kernel waits for memory once.  The
// projection adds in the same order as append_rows_kernel (an fma chain over
// d, then the parts in order).
template <int KVT, int KPT, int R, int DPER>
__global__ __launch_bounds__(256) void append_new_kernel(AppendArgs a) {
  constexpr int EB = Elem<KVT>::bytes;
  constexpr int PARTS = 256 / R;
  __shared__ float s_part[256];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int o = threadIdx.x % R, part = threadIdx.x / R;
  const int d0 = part * DPER;
  const char* src = reinterpret_cast<const char*>(a.k_new) + ((size_t(b) * a.n_new + j) * a.Hkv + h) * a.d_k * EB;
  const float* Pc = a.P + size_t(h) * a.d_k * R + o;
  float kv[DPER], pv[DPER];
#pragma unroll
  for (int i = 0; i < DPER; ++i) {
    if constexpr (KVT == 1) kv[i] = bf16_lo(uint32_t(reinterpret_cast<const uint16_t*>(src)[d0 + i]));
    else kv[i] = reinterpret_cast<const float*>(src)[d0 + i];
    pv[i] = Pc[size_t(d0 + i) * R];
  }
  const int n16k = a.d_k * EB / 16;
  const bool copy_v = !a.mla && a.v_new;
  const int n16v = copy_v ? a.d_v * EB / 16 : 0;
  const char* vsrc = copy_v ? reinterpret_cast<const char*>(a.v_new) + ((size_t(b) * a.n_new + j) * a.Hkv + h) * a.d_v * EB
                            : nullptr;
  uint4 kc16 = make_uint4(0u, 0u, 0u, 0u), vc16 = make_uint4(0u, 0u, 0u, 0u);
  if (int(threadIdx.x) < n16k) kc16 = load16(src + size_t(threadIdx.x) * 16);
  if (int(threadIdx.x) < n16v) vc16 = load16(vsrc + size_t(threadIdx.x) * 16);
  const int t = a.pos[b] + j;
  const bool ok = t >= 0 && t < a.t_max;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < DPER; ++i) acc = fmaf(kv[i], pv[i], acc);
  s_part[threadIdx.x] = acc;
  if (ok) {
    if (int(threadIdx.x) < n16k)
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.k_cache) + ((size_t(b) * a.t_max + t) * a.Hkv + h) * a.d_k * EB +
                                size_t(threadIdx.x) * 16) = kc16;
    if (int(threadIdx.x) < n16v)
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.v_cache) + ((size_t(b) * a.t_max + t) * a.Hkv + h) * a.d_v * EB +
                                size_t(threadIdx.x) * 16) = vc16;
  }
  __syncthreads();
  if (ok && int(threadIdx.x) < R) {
    float sum = 0.f;
    for (int pp = 0; pp < PARTS; ++pp) sum += s_part[pp * R + threadIdx.x];
    char* kprow = reinterpret_cast<char*>(a.kp) + ((size_t(b) * a.Hkv + h) * a.t_max + t) * R * Elem<KPT>::bytes;
    if constexpr (KPT == 1) reinterpret_cast<uint16_t*>(kprow)[threadIdx.x] = f32_to_bf16_rne(sum);
    else if constexpr (KPT == 2) reinterpret_cast<uint8_t*>(kprow)[threadIdx.x] = uint8_t(f32_to_e4m3_sat(sum));
    else reinterpret_cast<float*>(kprow)[threadIdx.x] = sum;
  }
}

// Few new rows of a wide key (the MLA latent row): one workgroup per row
// (append_wide_row).
template <int KVT, int KPT, int R, int D, int PARTS>
__global__ __launch_bounds__(R * PARTS) void append_wide_kernel(AppendArgs a) {
  __shared__ float s_part[R * PARTS];
  append_wide_row<KVT, KPT, R, D, PARTS>(a, blockIdx.x, blockIdx.y, blockIdx.z, s_part);
}

template <int KVT, int KPT>
static hipError_t dispatch_append_r(const AppendArgs& args, int r, dim3 grid, hipStream_t s) {
  if (args.mla && args.n_new <= kAppendRowsMax && args.k_new && args.d_k == kMlaDk) {
    dim3 g(args.n_new, grid.y, grid.z);
    if (r == 64) {
      hipLaunchKernelGGL((append_wide_kernel<KVT, KPT, 64, kMlaDk, 16>), g, dim3(1024), 0, s, args);
      return hipGetLastError();
    }
    if (r == 32) {
      hipLaunchKernelGGL((append_wide_kernel<KVT, KPT, 32, kMlaDk, 32>), g, dim3(1024), 0, s, args);
      return hipGetLastError();
    }
  }
  if (args.n_new <= kAppendRowsMax && args.k_new) {
    dim3 g(args.n_new, grid.y, grid.z);
    const int dper = args.d_k * r / 256;
    if (args.d_k * r % 256 == 0) {
      if (r == 32 && dper == 16) {
        hipLaunchKernelGGL((append_new_kernel<KVT, KPT, 32, 16>), g, dim3(256), 0, s, args);
        return hipGetLastError();
      }
      if (r == 64 && dper == 32) {
        hipLaunchKernelGGL((append_new_kernel<KVT, KPT, 64, 32>), g, dim3(256), 0, s, args);
        return hipGetLastError();
      }
      if (r == 16 && dper == 4) {
        hipLaunchKernelGGL((append_new_kernel<KVT, KPT, 16, 4>), g, dim3(256), 0, s, args);
        return hipGetLastError();
      }
      if (r == 32 && dper == 8) {
        hipLaunchKernelGGL((append_new_kernel<KVT, KPT, 32, 8>), g, dim3(256), 0, s, args);
        return hipGetLastError();
      }
    }
  }
  if (args.n_new <= kAppendRowsMax) {
    dim3 g(args.n_new, grid.y, grid.z);
    switch (r) {
      case 16: hipLaunchKernelGGL((append_rows_kernel<KVT, KPT, 16>), g, dim3(256), 0, s, args); break;
      case 32: hipLaunchKernelGGL((append_rows_kernel<KVT, KPT, 32>), g, dim3(256), 0, s, args); break;
      case 64: hipLaunchKernelGGL((append_rows_kernel<KVT, KPT, 64>), g, dim3(256), 0, s, args); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (r) {
    case 16: hipLaunchKernelGGL((append_kernel<KVT, KPT, 16>), grid, dim3(256), 0, s, args); break;
    case 32: hipLaunchKernelGGL((append_kernel<KVT, KPT, 32>), grid, dim3(256), 0, s, args); break;
    case 64: hipLaunchKernelGGL((append_kernel<KVT, KPT, 64>), grid, dim3(256), 0, s, args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_append(const jssa_desc& d, const void* k_new, const void* v_new, int n_new,
                         const int32_t* pos, const float* P, void* k_cache, void* v_cache,
                         void* kp_cache, hipStream_t s) {
  AppendArgs a;
  a.k_new = k_new; a.v_new = v_new; a.pos = pos; a.P = P;
  a.k_cache = k_cache; a.v_cache = v_cache; a.kp = kp_cache;
  a.n_new = n_new; a.Hkv = d.n_kv_heads; a.d_k = d.d_k; a.d_v = d.d_v; a.t_max = d.t_max;
  a.mla = d.layout == JSSA_LAYOUT_MLA;
  dim3 grid((n_new + 255) / 256, d.n_kv_heads, d.batch);
  const bool kvb = d.kv_dtype == JSSA_BF16, kpb = d.kp_dtype == JSSA_BF16;
  if (d.kp_dtype == JSSA_FP8_E4M3) {
    if (!kvb) return hipErrorInvalidValue;
    return dispatch_append_r<1, 2>(a, d.rank, grid, s);
  }
  if (kvb && kpb) return dispatch_append_r<1, 1>(a, d.rank, grid, s);
  if (kvb && !kpb) return dispatch_append_r<1, 0>(a, d.rank, grid, s);
  if (!kvb && kpb) return dispatch_append_r<0, 1>(a, d.rank, grid, s);
  return dispatch_append_r<0, 0>(a, d.rank, grid, s);
}

// Workspace zero-fill: a kernel rather than a memset so that it can be
// captured in a graph.
__global__ __launch_bounds__(256) void zero_kernel(char* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = size_t(gridDim.x) * 256;
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(p)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x < (bytes & 15)) p[n16 * 16 + threadIdx.x] = 0;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = (bytes / 16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, reinterpret_cast<char*>(p), bytes);
  return hipGetLastError();
}

// Diagnostic words of a workspace: copied out (plain loads: the calls that
// wrote them are earlier launches on the stream) and optionally cleared.
__global__ __launch_bounds__(64) void status_kernel(uint32_t* queue, uint32_t* out, int clear) {
  const int i = threadIdx.x;
  if (i < kStatusWords) {
    out[i] = queue[QW_ERR + i];
    if (clear) queue[QW_ERR + i] = 0u;
  }
}

hipError_t launch_status(uint32_t* queue, uint32_t* out, bool clear, hipStream_t s) {
  hipLaunchKernelGGL(status_kernel, dim3(1), dim3(64), 0, s, queue, out, clear ? 1 : 0);
  return hipGetLastError();
}

// The step's new K and V rows of a layer that keeps no scoring cache (its
// index lists come from another layer): one workgroup per sequence copies the
// token's Hkv rows of K, then of V, in 16-byte pieces (all of a sequence's
// rows of one token are contiguous in both layouts).
__global__ __launch_bounds__(256) void copy_new_kernel(const char* k_new, const char* v_new, const int32_t* pos,
                                                       char* k_cache, char* v_cache, int kb, int vb, int t_max) {
  const int b = blockIdx.x;
  const int t = pos[b];
  if (t < 0 || t >= t_max) return;
  const int nk = kb / 16, n = nk + vb / 16;
  for (int i = threadIdx.x; i < n; i += 256) {
    if (i < nk)
      *reinterpret_cast<uint4*>(k_cache + (size_t(b) * t_max + t) * kb + size_t(i) * 16) =
          load16(k_new + size_t(b) * kb + size_t(i) * 16);
    else
      *reinterpret_cast<uint4*>(v_cache + (size_t(b) * t_max + t) * vb + size_t(i - nk) * 16) =
          load16(v_new + size_t(b) * vb + size_t(i - nk) * 16);
  }
}

hipError_t launch_copy_new(const jssa_desc& d, const void* k_new, const void* v_new, const int32_t* pos,
                           void* k_cache, void* v_cache, hipStream_t s) {
  const int eb = d.kv_dtype == JSSA_BF16 ? 2 : 4;
  const bool mla = d.layout == JSSA_LAYOUT_MLA;
  const int kb = d.n_kv_heads * d.d_k * eb, vb = mla ? 0 : d.n_kv_heads * d.d_v * eb;
  if ((kb & 15) || (vb & 15) || d.batch <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_new_kernel, dim3(unsigned(d.batch)), dim3(256), 0, s, static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), pos, static_cast<char*>(k_cache), static_cast<char*>(v_cache),
                     kb, vb, d.t_max);
  return hipGetLastError();
}

}  // namespace jssa
