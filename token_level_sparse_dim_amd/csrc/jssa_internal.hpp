// Internal declarations shared by the host ABI layer and the HIP kernels of
// the gfx950 sparse-decode library: workspace layout, tiling constants and
// the launchers the ABI layer calls.  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "jssa.h"

namespace jssa {

// ---- tiling constants -------------------------------------------------------
constexpr int kScoreTile = 4096;     // candidate tokens per score workgroup
constexpr int kSelTile = 4096;       // keys per selection workgroup (must equal kScoreTile)
constexpr int kDigit1Bits = 12;      // first radix digit: key bits 31..20
constexpr int kDigit1Bins = 1 << kDigit1Bits;
constexpr int kMaxSelTiles = 4096;   // t_max <= kMaxSelTiles * kSelTile
constexpr int kAttnBlock = 64;       // tokens per attention inner block (per workgroup pass)
constexpr int kRowStateWords = 16;   // u32 words of per-row selection state

// per-row selection state (u32 words)
enum RowState : int {
  RS_MODE = 0,        // 0: select, 1: take every candidate, 2: nothing to select
  RS_D1 = 1,          // first-digit threshold bin
  RS_NEED1 = 2,       // how many keys with digit == D1 are still needed
  RS_KSTAR = 3,       // exact key of the k-th selected candidate
  RS_ISTAR = 4,       // ties at KSTAR are taken for indices <= ISTAR
  RS_NSCAN = 5,       // number of selected candidates
  RS_CAND_COUNT = 6,  // running count of first-digit candidates (zero on entry/exit)
  RS_TICKET_SCORE = 7,  // zero on entry/exit
  RS_TICKET_CAND = 8,   // zero on entry/exit
  RS_TICKET_ATTN = 9,   // zero on entry/exit
};

// ---- workspace layout ---------------------------------------------------------
// Every region starts 256-byte aligned.  The zero-on-entry regions are
// hist1, hist2 and the counter words of row_state; all other regions are
// fully written before they are read within a call.
struct Workspace {
  size_t hist1 = 0;      // u32 [rows][kDigit1Bins]      (zero on entry and exit)
  size_t hist2 = 0;      // u32 [rows][4096]             (zero on entry and exit)
  size_t row_state = 0;  // u32 [rows][kRowStateWords]
  size_t tile_gt = 0;    // u32 [rows][n_sel_tiles]
  size_t tile_off = 0;   // u32 [rows][n_sel_tiles]
  size_t cand = 0;       // u64 [rows][t_max]  (index << 32 | key)
  size_t part_acc = 0;   // f32 [rows][n_chunks][G][d_v]
  size_t part_ml = 0;    // f32 [rows][n_chunks][G][2]
  size_t scores = 0;     // f32 [rows][t_max]           (decode only)
  size_t idx = 0;        // i32 [rows][k+W]             (decode only)
  size_t n_sel = 0;      // i32 [rows]                  (decode only)
  size_t total = 0;
  int n_chunks = 0;      // attention chunks per row
  int chunk = 0;         // tokens per attention chunk
  int n_sel_tiles = 0;
};

// Layout for `op` (a jssa_op).  Returns false if the descriptor is invalid.
bool workspace_layout(const jssa_desc& d, int op, Workspace* ws);

// ---- launchers (return hipSuccess or the launch error) -------------------------
hipError_t launch_append(const jssa_desc& d, const void* k_new, const void* v_new, int n_new,
                         const int32_t* pos, const float* P, void* k_cache, void* v_cache,
                         void* kp_cache, hipStream_t s);

// Scores for every candidate; when `ws_base` is non-null also builds the
// first-digit histogram and the per-row threshold state used by selection.
hipError_t launch_score(const jssa_desc& d, const void* q, const float* P, const void* kp,
                        const int32_t* seq_lens, float* scores, char* ws_base, const Workspace& ws,
                        hipStream_t s);

// First-digit histogram and threshold of caller-provided scores.
hipError_t launch_hist(const jssa_desc& d, const float* scores, const int32_t* seq_lens,
                       char* ws_base, const Workspace& ws, hipStream_t s);

// Selection from fp32 scores: histogram (unless `hist_done`), candidates and
// exact resolution, emission of indices in ascending order plus the window.
hipError_t launch_topk(const jssa_desc& d, const float* scores, const int32_t* seq_lens,
                       int32_t* idx, int32_t* n_sel, char* ws_base, const Workspace& ws,
                       bool hist_done, hipStream_t s, hipEvent_t after_select = nullptr);

// Attention over idx (indexed) or over every cached token (idx == nullptr).
hipError_t launch_attention(const jssa_desc& d, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* idx, const int32_t* n_sel,
                            const int32_t* seq_lens, void* out, float* lse, char* ws_base,
                            const Workspace& ws, hipStream_t s);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace jssa
