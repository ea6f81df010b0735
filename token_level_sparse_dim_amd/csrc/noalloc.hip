// jssa_decode_step_static: the one-call decode step with its intermediates in
// a static device array instead of a caller workspace, for callers that cannot
// allocate device memory.
//
// The array is this file's `scratch`.  Host code never passes the array's name
// to a kernel or copy (on the host it only names a stand-in): the device
// address is taken once per device, with that device current, through
// hipGetSymbolAddress, and kept in `g_scratch`.
//
// Layout inside the array: the workspace layout of the decode for the call's
// descriptor, except that the per-row state (whose words must be zero on entry
// and are left zero by every call) is reserved for JSSA_STATIC_SCRATCH_ROWS
// rows whatever the descriptor, so a later call with more rows never finds
// another call's data where its counters live.  The queue words (also zero on
// entry, or sticky diagnostics) sit at offset 0 in every layout.  Both regions
// are zeroed once, by the first call on a device; every other region is
// written before it is read within a call.
#include <mutex>

#include "jssa_internal.hpp"

static __device__ __align__(256) char scratch[JSSA_STATIC_SCRATCH_BYTES];

namespace jssa {
namespace {

constexpr size_t kScratchBytes = JSSA_STATIC_SCRATCH_BYTES;
constexpr int kScratchRows = JSSA_STATIC_SCRATCH_ROWS;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
char* g_scratch[kMaxDevices] = {};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Bytes at the start of the array that hold the queue and the reserved row
// state (zero on entry).
constexpr size_t kZeroBytes = 256 + size_t(kScratchRows) * kRowStateWords * 4;

// This device's address of `scratch`; the first call on a device also zeroes
// the counter regions on `s`.  nullptr if the device or the symbol is not
// available (the HIP error in *err).
char* device_scratch(hipStream_t s, hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(::scratch));
    if (*err != hipSuccess || !p) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    *err = launch_zero(p, kZeroBytes, s);
    if (*err != hipSuccess) return nullptr;
    g_scratch[dev] = static_cast<char*>(p);
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace jssa

using namespace jssa;

extern "C" int32_t jssa_decode_step_static(const jssa_desc* desc, const void* k_new, const void* v_new,
                                           const int32_t* pos, const void* q, const float* P, void* kp_cache,
                                           void* k_cache, void* v_cache, const int32_t* seq_lens, void* out,
                                           float* lse, int32_t* idx_out, int32_t* n_sel_out, void* stream) {
  if (!desc) return JSSA_ERR_INVALID_ARG;
  const bool mla = desc->layout == JSSA_LAYOUT_MLA;
  const NewToken nt{k_new, mla ? nullptr : v_new, pos, k_cache, v_cache, kp_cache};
  const int32_t st = check_decode_args(desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, idx_out,
                                       n_sel_out, &nt, nullptr);
  if (st != JSSA_OK) return st;
  Workspace lay;
  if (!workspace_layout(*desc, JSSA_OP_DECODE, &lay)) return JSSA_ERR_INVALID_ARG;
  if (!lay.pipe) return JSSA_ERR_UNSUPPORTED;  // the fused decode shapes only
  const size_t rows = size_t(desc->batch) * desc->n_kv_heads;
  if (rows > size_t(kScratchRows)) return JSSA_ERR_TOO_LARGE;
  // the regions after the row state move past its reserved size
  const size_t state_end = lay.row_state + round256(rows * kRowStateWords * 4);
  if (lay.queue != 0 || lay.row_state != 256 || state_end > kZeroBytes) return JSSA_ERR_UNSUPPORTED;
  Workspace fixed = rebase_workspace(lay, kZeroBytes - state_end, lay.queue);
  fixed.row_state = lay.row_state;
  if (fixed.total > kScratchBytes) return JSSA_ERR_TOO_LARGE;
  hipError_t err = hipSuccess;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = device_scratch(s, &err);
  if (!base) return JSSA_ERR_HIP;
  return decode_launch(desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, idx_out, n_sel_out, base, fixed,
                       &nt, nullptr, stream);
}
