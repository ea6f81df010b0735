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
// Compile-time tuning knobs (defaults are the measured choices on MI355X).
#ifndef JSSA_SCORE_TILE
#define JSSA_SCORE_TILE 4096
#endif
#ifndef JSSA_SCORE_UNROLL
#define JSSA_SCORE_UNROLL 4
#endif
#ifndef JSSA_ATTN_UNROLL
#define JSSA_ATTN_UNROLL 4
#endif
constexpr int kScoreTile = JSSA_SCORE_TILE;  // candidate tokens per score workgroup
constexpr int kSelTile = 4096;               // keys per selection workgroup
constexpr int kSubTile = 1024;               // tokens per tile of the fused selection's candidate slots
constexpr int kDigit1Bits = 12;      // first radix digit: key bits 31..20
constexpr int kDigit1Bins = 1 << kDigit1Bits;
constexpr int kMaxSelTiles = 4096;   // t_max <= kMaxSelTiles * kSelTile
constexpr int kAttnBlock = 64;       // tokens per attention inner block (per workgroup pass)
constexpr int kRowStateWords = 16;   // u32 words of per-row selection state
constexpr int kCandPad = 128;        // candidate slots past the last row (read, never used)
constexpr int kMaxPipeChunk = 1024;  // attention chunk limit of the fused decode
// MLA layout: shared latent rows of kMlaDk elements, values = first kMlaDv
constexpr int kMlaDk = 576;
constexpr int kVoteChunk = 2048;    // candidates per partial of the head-shared vote
constexpr int kVoteMaxHeads = 64;   // KV heads the vote merges in shared memory
constexpr int kMlaDv = 512;
constexpr int kMlaScoreTile = 1024;  // candidate tokens per MLA score workgroup
constexpr int kMlaHeadGroup = 32;    // query heads per MLA attention workgroup

// per-row state (u32 words).  The tickets and the ready flag are zero on
// entry and are left zero by every call.
enum RowState : int {
  RS_D1 = 1,            // first-digit (key bits 31..20) threshold bin
  RS_NEED1 = 2,         // keys still needed from bin D1 (k minus the count above it)
  RS_KSTAR = 3,         // key of the k-th selected candidate
  RS_ISTAR = 4,         // keys equal to KSTAR are selected for indices <= ISTAR
  RS_NCAND = 5,         // candidates of the row (keys in or above bin D1)
  RS_TICKET_SCORE = 7,  // arrivals of score / histogram workgroups
  RS_READY = 8,         // selection of the row published (set by resolve, cleared by attention)
  RS_TICKET_ATTN = 9,   // arrivals of attention chunks
};

// Queue words of a workspace (the first region of every layout).  QW_NEXT and
// QW_DONE are the work queue of the resolve + attention launch (zero on entry
// and exit); the others are sticky diagnostics that accumulate over calls
// until jssa_workspace_status clears them.
enum QueueWord : int {
  QW_NEXT = 0,    // next item of the resolve + attention launch
  QW_DONE = 1,    // finished items of that launch
  QW_ERR = 2,     // nonzero: a bounded wait gave up (that call's results are unreliable)
  QW_REDO = 3,    // rows re-selected exactly (the sampled threshold admitted fewer than k tokens)
  QW_RANGE = 4,   // fused scans that split the score work into ranges across rows (fewer workgroups than rows)
  QW_BIG = 5,     // rows whose candidates exceeded shared memory (cut in global memory)
};
constexpr int kQueueWords = 64;
constexpr int kStatusWords = 4;  // words jssa_workspace_status reports: QW_ERR .. QW_ERR + 3

// ---- workspace layout ---------------------------------------------------------
// Every region starts 256-byte aligned.  The zero-on-entry regions are
// hist1, row_state and queue; all other regions are fully written before
// they are read within a call.
struct Workspace {
  size_t hist1 = 0;      // u32 [rows][kDigit1Bins]      (zero on entry and exit)
  size_t row_state = 0;  // u32 [rows][kRowStateWords]
  size_t queue = 0;      // u32 [kQueueWords]            (zero on entry and exit)
  size_t tile_cnt = 0;   // u32 [rows][n_sel_tiles]      candidates per selection tile
  size_t tile_off = 0;   // u32 [rows][n_sel_tiles]      first output position of each tile
  size_t cand_base = 0;  // u32 [rows][n_sel_tiles]      first candidate of each tile (concatenated)
  size_t cand = 0;       // u64 [rows][t_max]  (index << 32 | key), in tile slots of kSelTile
  size_t part_acc = 0;   // f32 [rows][n_chunks][G][d_v]
  size_t part_ml = 0;    // f32 [rows][n_chunks][G][2]
  size_t scores = 0;     // f32 [rows][t_max]           (decode only)
  size_t idx = 0;        // i32 [rows][k+W]             (decode only)
  size_t n_sel = 0;      // i32 [rows]                  (decode only)
  size_t qfrag = 0;      // bf16 projected-query MFMA fragments (MLA score)
  size_t pipe_qp = 0;    // f32 [rows][G][r] the rows' projected queries (fused decode)
  size_t vote_part = 0;  // f32 [rows][vote chunks][2]  (head-shared voting)
  size_t vote = 0;       // f32 [B][t_max]              the sequences' votes
  size_t vote_idx = 0;   // i32 [B][k+W]                the shared lists
  size_t vote_nsel = 0;  // i32 [B]
  size_t vote_range = 0; // u32 [B][2]                  (zero on entry and exit)
  size_t vote_topk = 0;  // the top-k workspace of the one-head vote descriptor
  size_t total = 0;
  int n_chunks = 0;      // attention chunks per row
  int chunk = 0;         // tokens per attention chunk
  int n_sel_tiles = 0;
  // fused decode (one persistent launch): available for the shapes it is built
  // for; score items of pipe_ts tokens, pipe_tiles per row (tile_cnt and the
  // candidate slots are shared with the staged path and sized for both)
  bool pipe = false;
  int pipe_ts = 0, pipe_tiles = 0, pipe_chunk = 0, pipe_n_chunks = 0;
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

// Candidate pass of the selection: every key in or above the first-digit
// threshold bin, written in token order to its tile's slot.
// sub_tiles: slots and counts per kSubTile tokens (the fused selection's
// tiles) instead of per kSelTile
hipError_t launch_candidates(const jssa_desc& d, const float* scores, const int32_t* seq_lens,
                             char* ws_base, const Workspace& ws, hipStream_t s, bool sub_tiles = false);

// One launch with a work queue: a resolve item per row (exact k-th key, tie
// cut, emission of idx / n_sel in ascending order plus the window), and, when
// `attend`, the attention chunks of every row, each waiting for its row's
// resolve.  Without `resolve`, idx / n_sel are inputs.  idx == nullptr with
// `attend` and no `resolve` selects the dense path (every t < seq_lens[b]).
hipError_t launch_resolve_attend(const jssa_desc& d, bool resolve, bool attend, const void* q,
                                 const void* k_cache, const void* v_cache, int32_t* idx,
                                 int32_t* n_sel, const int32_t* seq_lens, void* out, float* lse,
                                 char* ws_base, const Workspace& ws, hipStream_t s);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
// Copies the workspace's diagnostic words (QW_ERR ..) to `out` and, with
// `clear`, zeroes them (a kernel: safe inside graph capture).
hipError_t launch_status(uint32_t* queue, uint32_t* out, bool clear, hipStream_t s);
// A layout whose regions are shifted by `delta` bytes except the queue, which
// is placed at `queue`: a nested workspace that reports its diagnostics in
// its parent's queue.
Workspace rebase_workspace(const Workspace& w, size_t delta, size_t queue);
// Head-shared soft voting (vote.hip): the vote of every KV head's scores, its
// top-k (with the one-head descriptor vote_desc(d)) and the list copied to
// every KV head.
jssa_desc vote_desc(const jssa_desc& d);
hipError_t launch_vote_select(const jssa_desc& d, const float* scores, const int32_t* seq_lens, int32_t* idx,
                              int32_t* n_sel, char* ws_base, const Workspace& ws, hipStream_t s);
// Packs the selected K (and V) rows into [B, topk + window, Hkv, d] buffers
// (gather.hip); lens_out[b] = n_sel[b, 0] if given.
hipError_t launch_gather_kv(const jssa_desc& d, const void* k_cache, const void* v_cache, const int32_t* idx,
                            const int32_t* n_sel, void* k_out, void* v_out, int32_t* lens_out, hipStream_t s);

// MLA scoring on the matrix cores: the query projection into ws.qfrag, then
// the score scan that reads it; with `hist` the scan also builds the
// first-digit histogram and threshold state.
hipError_t launch_mla_qproj(const jssa_desc& d, const void* q, const float* P, char* ws_base, const Workspace& ws,
                            hipStream_t s);
bool mla_prep_fusable(const jssa_desc& d);
hipError_t launch_mla_prep(const jssa_desc& d, const void* k_new, const int32_t* pos, const float* P,
                           void* k_cache, void* kp_cache, const void* q, char* ws_base, const Workspace& ws,
                           hipStream_t s);
hipError_t launch_mla_scan(const jssa_desc& d, const void* kp, const int32_t* seq_lens, float* scores, bool hist,
                           char* ws_base, const Workspace& ws, hipStream_t s,
                           void* const* ev = nullptr);

// MLA attention over idx / n_sel (idx == nullptr: every t < seq_lens[b]) in
// chunks of ws.chunk rows, then the log-sum-exp merge of the chunks.
hipError_t launch_mla_attend(const jssa_desc& d, const void* q, const void* k_cache, const int32_t* idx,
                             const int32_t* n_sel, const int32_t* seq_lens, void* out, float* lse,
                             char* ws_base, const Workspace& ws, hipStream_t s);

// Fused decode: whether a build exists for the descriptor's shape, its tile
// size, tiles per row and attention chunk (tokens).
bool pipeline_layout(const jssa_desc& d, int* ts, int* n_tiles, int* chunk);
// The dense decode on the fused shapes: the decode's attention parts over
// every position, `chunk` positions per part, n_chunks parts per row.
bool dense_pipe_layout(const jssa_desc& d, int* chunk, int* n_chunks);

// The step's new token (one row per sequence and KV head, at t = pos[b]) and
// the caches it is written to, for a decode that appends it itself.
struct NewToken {
  const void* k_new;
  const void* v_new;
  const int32_t* pos;
  void* k_cache;
  void* v_cache;
  void* kp_cache;
};

// The whole decode step in two launches (the scan with sampled-threshold
// candidate emission, preceded by a sample launch when the rows outnumber the
// resident scan workgroups; then selection, attention and merge in one
// launch); requires ws.pipe.  With `ev` (four events): [0] and [1] the scan
// kernel's own start and end, [2] after the select/attend launch, [3] right
// after.  With `nt`, the scan launch also appends the new token (the caches in
// `nt` are the decode's caches).
hipError_t launch_pipeline(const jssa_desc& d, const void* q, const float* P, const void* kp,
                           const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                           float* lse, int32_t* idx, int32_t* n_sel, char* ws_base, const Workspace& ws,
                           const NewToken* nt, void* const* ev, hipStream_t s);
// The exact selection of each row from the candidate pass's per-1024-token
// slots (the MLA decode), one 1024-thread workgroup per row.
hipError_t launch_select_rows(const jssa_desc& d, const int32_t* seq_lens, int32_t* idx, int32_t* n_sel,
                              char* ws_base, const Workspace& ws, hipStream_t s);
// The fused decode's attention parts (and their in-launch merge) on
// caller-provided index lists (stride topk + window), with the decode
// workspace (pipeline shapes only).
hipError_t launch_pipe_dense(const jssa_desc& d, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, void* out, float* lse, char* ws_base, const Workspace& ws,
                             hipStream_t s);
hipError_t launch_pipe_attend(const jssa_desc& d, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* idx, const int32_t* n_sel, void* out, float* lse, char* ws_base,
                              const Workspace& ws, hipStream_t s);
// Host-side checks of a decode's arguments except the workspace (abi.cpp),
// and the decode's launches on a workspace of layout `lay` (nt: the step's new
// token, appended first; ev: four stage events or null).
int32_t check_decode_args(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                          const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                          float* lse, int32_t* idx_out, int32_t* n_sel_out, const NewToken* nt, void* const* ev);
int32_t decode_launch(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                      const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out, float* lse,
                      int32_t* idx_out, int32_t* n_sel_out, char* base, const Workspace& lay, const NewToken* nt,
                      void* const* ev, void* stream);
// Copies the step's new K (and V) rows, [B, 1, Hkv, d], to t = pos[b] of the
// caches (no projection); rows with t outside [0, t_max) are skipped.
hipError_t launch_copy_new(const jssa_desc& d, const void* k_new, const void* v_new, const int32_t* pos,
                           void* k_cache, void* v_cache, hipStream_t s);

}  // namespace jssa
