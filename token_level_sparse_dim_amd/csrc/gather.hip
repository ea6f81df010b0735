// Gather of the selected K/V rows into packed buffers: the "gather-then-
// attend" baseline the pages compare gather-free execution against (JSSA
// summary section 2.2 and Figure 2(b): gathering the selected entries is a
// large share of the sparse latency; section 4.7: with the same selected
// tokens, gather-free execution roughly doubles the attention-stage speedup).
// The packed rows keep the cache's [B, S, Hkv, d] layout, so the dense decode
// attends over them with seq_lens = the selection counts.
#include "jssa_device.hpp"
#include "jssa_internal.hpp"

namespace jssa {

struct GatherArgs {
  const char* k;
  const char* v;  // nullptr: MLA (the value is a prefix of the key row)
  const int32_t* idx;
  const int32_t* n_sel;
  char* k_out;
  char* v_out;
  int32_t* lens_out;
  int Hkv, t_max, S, k_row, v_row;  // S = index-list stride; row bytes of K and V
};

// 16 rows per workgroup, 16 lanes per row, 16-byte pieces.  Indices are
// clamped into [0, t_max) as the attention kernels clamp them; list entries
// past n_sel are not read and their packed rows are not written.
__global__ __launch_bounds__(256) void gather_kv_kernel(GatherArgs a) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int row = blockIdx.x * 16 + int(threadIdx.x >> 4), lane = threadIdx.x & 15;
  const int row_id = b * a.Hkv + h;
  int n = a.n_sel[row_id];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  if (a.lens_out && h == 0 && blockIdx.x == 0 && threadIdx.x == 0) a.lens_out[b] = n;
  if (row >= n) return;
  int t = a.idx[size_t(row_id) * a.S + row];
  t = t < 0 ? 0 : (t >= a.t_max ? a.t_max - 1 : t);
  const size_t src = (size_t(b) * a.t_max + t) * a.Hkv + h;
  const size_t dst = (size_t(b) * a.S + row) * a.Hkv + h;
  for (int p = lane * 16; p < a.k_row; p += 256)
    *reinterpret_cast<uint4*>(a.k_out + dst * a.k_row + p) = load16_nt(a.k + src * a.k_row + p);
  if (a.v)
    for (int p = lane * 16; p < a.v_row; p += 256)
      *reinterpret_cast<uint4*>(a.v_out + dst * a.v_row + p) = load16_nt(a.v + src * a.v_row + p);
}

hipError_t launch_gather_kv(const jssa_desc& d, const void* k_cache, const void* v_cache, const int32_t* idx,
                            const int32_t* n_sel, void* k_out, void* v_out, int32_t* lens_out, hipStream_t s) {
  GatherArgs a;
  const int eb = d.kv_dtype == JSSA_BF16 ? 2 : 4;
  const bool mla = d.layout == JSSA_LAYOUT_MLA;
  a.k = static_cast<const char*>(k_cache);
  a.v = mla ? nullptr : static_cast<const char*>(v_cache);
  a.idx = idx; a.n_sel = n_sel;
  a.k_out = static_cast<char*>(k_out);
  a.v_out = mla ? nullptr : static_cast<char*>(v_out);
  a.lens_out = lens_out;
  a.Hkv = d.n_kv_heads; a.t_max = d.t_max; a.S = d.topk + d.window;
  a.k_row = d.d_k * eb; a.v_row = d.d_v * eb;
  dim3 grid((a.S + 15) / 16, d.n_kv_heads, d.batch);
  hipLaunchKernelGGL(gather_kv_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace jssa
