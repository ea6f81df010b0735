// The new-row append shared by the append launches and the MLA decode's
// first launch (JSSA summary section E.1: each newly generated key is
// projected into the scoring cache, Kp = K P).
#pragma once

#include "jssa_device.hpp"
#include "jssa_internal.hpp"

namespace jssa {

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* pos;
  const float* P;
  void* k_cache;
  void* v_cache;
  void* kp;
  int n_new, Hkv, d_k, d_v, t_max;
  int mla;
};

// New row j of KV head h of sequence b for a wide key (the MLA latent row,
// D = 576), by one workgroup of R * PARTS = 1024 threads: thread (o, part)
// runs an fma chain over its D / PARTS slice of d with every load of the
// slice requested at once; the parts are then summed in order.  (A
// 256-thread workgroup walks 144 dependent basis loads per thread.)  s_part:
// R * PARTS floats of shared memory.
template <int KVT, int KPT, int R, int D, int PARTS>
__device__ __forceinline__ void append_wide_row(const AppendArgs& a, int j, int h, int b, float* s_part) {
  constexpr int EB = Elem<KVT>::bytes, NT = R * PARTS, DPER = D / PARTS;
  static_assert(D % PARTS == 0 && NT <= 1024, "slices");
  const int o = threadIdx.x % R, part = threadIdx.x / R;
  const int d0 = part * DPER;
  const char* src = reinterpret_cast<const char*>(a.k_new) + ((size_t(b) * a.n_new + j) * a.Hkv + h) * D * EB;
  const float* Pc = a.P + size_t(h) * D * R + o;
  float kv[DPER], pv[DPER];
#pragma unroll
  for (int i = 0; i < DPER; ++i) {
    if constexpr (KVT == 1) kv[i] = bf16_lo(uint32_t(reinterpret_cast<const uint16_t*>(src)[d0 + i]));
    else kv[i] = reinterpret_cast<const float*>(src)[d0 + i];
    pv[i] = Pc[size_t(d0 + i) * R];
  }
  constexpr int N16 = D * EB / 16;
  uint4 kc16 = make_uint4(0u, 0u, 0u, 0u);
  if (int(threadIdx.x) < N16) kc16 = load16(src + size_t(threadIdx.x) * 16);
  const int t = a.pos[b] + j;
  const bool ok = t >= 0 && t < a.t_max;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < DPER; ++i) acc = fmaf(kv[i], pv[i], acc);
  s_part[threadIdx.x] = acc;
  if (ok && int(threadIdx.x) < N16)
    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.k_cache) + ((size_t(b) * a.t_max + t) * a.Hkv + h) * D * EB +
                              size_t(threadIdx.x) * 16) = kc16;
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

}  // namespace jssa
