// Host side of the C ABI declared in include/jssa.h: argument validation,
// workspace sizing and launch sequencing.  No entry point allocates, frees or
// synchronises; every check happens before the first launch.
#include <math.h>
#include <string.h>

#include "jssa_internal.hpp"

using jssa::Workspace;

namespace {

constexpr size_t kAlignWs = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t to_status(hipError_t e) { return e == hipSuccess ? JSSA_OK : JSSA_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Attention chunking: about 256 workgroups (one per CU) for the indexed path,
// which measured best for 512-byte K/V rows on MI355X; about 1024 for the dense
// path.  Chunks are multiples of 64 tokens.
void attn_chunking(int rows, int64_t n_max, bool indexed, int* chunk, int* n_chunks) {
  const int64_t lo = indexed ? 128 : 256;
  const int64_t hi = indexed ? 1024 : 8192;
  const int64_t target = indexed ? 256 : 1024;
  int64_t c = (n_max * rows + target - 1) / target;
  c = (c + 63) / 64 * 64;
  if (c < lo) c = lo;
  if (c > hi) c = hi;
  *chunk = int(c);
  *n_chunks = int((n_max + c - 1) / c);
  if (*n_chunks < 1) *n_chunks = 1;
}

// MLA attention chunking: workgroups are (sequence, 32-head group, chunk);
// about 256 of them for the indexed path (one per CU: each holds a whole CU's
// registers) and 1024 for the dense path.  Chunks are multiples of 64 rows.
void mla_chunking(int batch, int groups, int64_t n_max, bool indexed, int* chunk, int* n_chunks) {
  const int64_t target = indexed ? 256 : 1024;
  const int64_t hi = indexed ? 2048 : 8192;
  int64_t c = (n_max * batch * groups + target - 1) / target;
  c = (c + 63) / 64 * 64;
  if (c < 64) c = 64;
  if (c > hi) c = hi;
  *chunk = int(c);
  *n_chunks = int((n_max + c - 1) / c);
  if (*n_chunks < 1) *n_chunks = 1;
}

}  // namespace

namespace jssa {

// Validation shared by every entry point.  op: 0 = append/score, else a jssa_op.
static int32_t check(const jssa_desc* d, int op) {
  if (!d) return JSSA_ERR_INVALID_ARG;
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1) return JSSA_ERR_INVALID_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return JSSA_ERR_INVALID_ARG;
  if (d->t_max < 1 || d->t_max > kMaxSelTiles * kSelTile) return JSSA_ERR_INVALID_ARG;
  if (d->topk < 0 || d->window < 0) return JSSA_ERR_INVALID_ARG;
  const bool selects = op == JSSA_OP_TOPK || op == JSSA_OP_ATTN || op == JSSA_OP_DECODE || op == JSSA_OP_VOTE;
  if (selects && int64_t(d->topk) + d->window < 1) return JSSA_ERR_INVALID_ARG;
  if (int64_t(d->topk) + d->window > (int64_t(1) << 30)) return JSSA_ERR_INVALID_ARG;
  if (d->kv_dtype != JSSA_F32 && d->kv_dtype != JSSA_BF16) return JSSA_ERR_INVALID_ARG;
  if (d->kp_dtype != JSSA_F32 && d->kp_dtype != JSSA_BF16 && d->kp_dtype != JSSA_FP8_E4M3)
    return JSSA_ERR_INVALID_ARG;
  if (d->out_dtype != JSSA_F32 && d->out_dtype != JSSA_BF16) return JSSA_ERR_INVALID_ARG;
  if (d->reduce != JSSA_REDUCE_MAX && d->reduce != JSSA_REDUCE_MEAN) return JSSA_ERR_INVALID_ARG;
  if (d->layout != JSSA_LAYOUT_GQA && d->layout != JSSA_LAYOUT_MLA) return JSSA_ERR_INVALID_ARG;
  if (!isfinite(d->scale)) return JSSA_ERR_INVALID_ARG;
  if (d->d_k < 1 || d->d_v < 1 || d->rank < 1 || d->rank > d->d_k) return JSSA_ERR_INVALID_ARG;
  if (d->rank != 16 && d->rank != 32 && d->rank != 64) return JSSA_ERR_UNSUPPORTED;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (op == JSSA_OP_VOTE && (d->layout != JSSA_LAYOUT_GQA || d->n_kv_heads > kVoteMaxHeads))
    return JSSA_ERR_UNSUPPORTED;  // (MLA has one index set per sequence already)
  if (d->layout == JSSA_LAYOUT_MLA) {
    // one latent row per token, the value is a prefix of it
    if (d->n_kv_heads != 1 || d->d_v > d->d_k) return JSSA_ERR_INVALID_ARG;
    if (d->d_k != kMlaDk || d->d_v != kMlaDv) return JSSA_ERR_UNSUPPORTED;
    if (d->rank != 32 && d->rank != 64) return JSSA_ERR_UNSUPPORTED;
    if (d->kv_dtype != JSSA_BF16 || d->kp_dtype != JSSA_BF16) return JSSA_ERR_UNSUPPORTED;
    if (d->n_q_heads != 64 && d->n_q_heads != 128) return JSSA_ERR_UNSUPPORTED;
    return JSSA_OK;
  }
  if (d->d_k != d->d_v) return JSSA_ERR_UNSUPPORTED;
  if (d->d_k != 64 && d->d_k != 128) return JSSA_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return JSSA_ERR_UNSUPPORTED;
  // FP8 projected keys: scored on the matrix cores (bf16 q/K/V, rank 32 or 64)
  if (d->kp_dtype == JSSA_FP8_E4M3 && (d->kv_dtype != JSSA_BF16 || (d->rank != 32 && d->rank != 64)))
    return JSSA_ERR_UNSUPPORTED;
  return JSSA_OK;
}

bool workspace_layout(const jssa_desc& d, int op, Workspace* ws) {
  if (check(&d, op) != JSSA_OK) return false;
  *ws = Workspace();
  const size_t rows = size_t(d.batch) * d.n_kv_heads;
  const int G = d.n_q_heads / d.n_kv_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, kAlignWs);
    return at;
  };
  const bool mla = d.layout == JSSA_LAYOUT_MLA;
  ws->n_sel_tiles = (d.t_max + kSelTile - 1) / kSelTile;
  int pipe_chunk = 0;
  // fused-build shapes: the decode, and the stand-alone indexed attention (which
  // runs the decode's attention and merge launches), use the pipeline's chunking
  if ((op == JSSA_OP_DECODE || op == JSSA_OP_ATTN) && pipeline_layout(d, &ws->pipe_ts, &ws->pipe_tiles, &pipe_chunk)) {
    const int64_t n_max = int64_t(d.topk) + d.window;
    ws->pipe = true;
    ws->pipe_chunk = pipe_chunk;
    ws->pipe_n_chunks = int((n_max + pipe_chunk - 1) / pipe_chunk);
  }
  if (op == JSSA_OP_DENSE && dense_pipe_layout(d, &ws->pipe_chunk, &ws->pipe_n_chunks)) ws->pipe = true;
  // the fused decode uses its own tile counts and candidate slots only; the
  // staged selection also needs the first-digit histogram and tile tables
  const bool staged = op == JSSA_OP_TOPK || (op == JSSA_OP_DECODE && !ws->pipe);
  // the MLA decode's candidate pass counts per kSubTile tokens (its selection
  // is the fused decode's); the staged top-k per kSelTile
  const int cnt_tiles = !staged ? ws->pipe_tiles
                        : (mla && op == JSSA_OP_DECODE) ? ws->n_sel_tiles * (kSelTile / kSubTile)
                                                        : ws->n_sel_tiles;
  ws->queue = take(kQueueWords * 4);  // first: jssa_workspace_status finds it at offset 0
  ws->row_state = take(rows * kRowStateWords * 4);
  if (ws->pipe) ws->pipe_qp = take(rows * size_t(G) * d.rank * 4);
  if (op == JSSA_OP_TOPK || op == JSSA_OP_DECODE) {
    if (staged) ws->hist1 = take(rows * kDigit1Bins * 4);
    ws->tile_cnt = take(rows * cnt_tiles * 4);
    if (staged) {
      ws->tile_off = take(rows * ws->n_sel_tiles * 4);
      ws->cand_base = take(rows * ws->n_sel_tiles * 4);
    }
    ws->cand = take((rows * size_t(d.t_max) + kCandPad) * 8);
  }
  if (op == JSSA_OP_ATTN || op == JSSA_OP_DECODE || op == JSSA_OP_DENSE) {
    const bool indexed = op != JSSA_OP_DENSE;
    const int64_t n_max = indexed ? int64_t(d.topk) + d.window : d.t_max;
    if (mla) mla_chunking(d.batch, d.n_q_heads / kMlaHeadGroup, n_max, indexed, &ws->chunk, &ws->n_chunks);
    else attn_chunking(int(rows), n_max, indexed, &ws->chunk, &ws->n_chunks);
    const int part_chunks = ws->pipe_n_chunks > ws->n_chunks ? ws->pipe_n_chunks : ws->n_chunks;
    ws->part_acc = take(rows * part_chunks * size_t(G) * d.d_v * 4);
    ws->part_ml = take(rows * part_chunks * size_t(G) * 2 * 4);
  }
  if (op == JSSA_OP_DECODE) {
    if (staged) ws->scores = take(rows * size_t(d.t_max) * 4);
    ws->idx = take(rows * (size_t(d.topk) + d.window) * 4);
    ws->n_sel = take(rows * 4);
  }
  if (mla && (op == JSSA_OP_SCORE || op == JSSA_OP_DECODE)) {
    const size_t mt = d.reduce == JSSA_REDUCE_MEAN ? 1 : size_t(d.n_q_heads) / 16;
    ws->qfrag = take(size_t(d.batch) * mt * (d.rank / 32) * 2 * 64 * 16);
  }
  if (op == JSSA_OP_VOTE) {
    const size_t n_vchunks = (size_t(d.t_max) + kVoteChunk - 1) / kVoteChunk;
    ws->vote_part = take(rows * n_vchunks * 2 * 4);
    ws->vote = take(size_t(d.batch) * d.t_max * 4);
    ws->vote_idx = take(size_t(d.batch) * (size_t(d.topk) + d.window) * 4);
    ws->vote_nsel = take(size_t(d.batch) * 4);
    ws->vote_range = take(size_t(d.batch) * 2 * 4);
    Workspace lt;
    if (!workspace_layout(vote_desc(d), JSSA_OP_TOPK, &lt)) return false;
    ws->vote_topk = take(lt.total);
  }
  ws->total = off;
  return true;
}

Workspace rebase_workspace(const Workspace& w, size_t delta, size_t queue) {
  Workspace r = w;
  for (size_t* f : {&r.hist1, &r.row_state, &r.tile_cnt, &r.tile_off, &r.cand_base, &r.cand, &r.part_acc,
                    &r.part_ml, &r.scores, &r.idx, &r.n_sel, &r.qfrag, &r.pipe_qp, &r.vote_part, &r.vote,
                    &r.vote_idx, &r.vote_nsel, &r.vote_range, &r.vote_topk})
    *f += delta;
  r.queue = queue;
  r.total = w.total + delta;
  return r;
}

static int32_t check_ws(const jssa_desc& d, int op, void* ws, size_t ws_bytes, Workspace* lay) {
  if (!workspace_layout(d, op, lay)) return JSSA_ERR_INVALID_ARG;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlignWs) != 0 || ws_bytes < lay->total)
    return JSSA_ERR_WORKSPACE;
  return JSSA_OK;
}

}  // namespace jssa

using namespace jssa;

#define JSSA_TRY(expr)            \
  do {                            \
    const int32_t st_ = (expr);   \
    if (st_ != JSSA_OK) return st_; \
  } while (0)

extern "C" {

int32_t jssa_abi_version(void) { return JSSA_ABI_VERSION; }

const char* jssa_status_str(int32_t s) {
  switch (s) {
    case JSSA_OK: return "JSSA_OK";
    case JSSA_ERR_INVALID_ARG: return "JSSA_ERR_INVALID_ARG";
    case JSSA_ERR_UNSUPPORTED: return "JSSA_ERR_UNSUPPORTED";
    case JSSA_ERR_WORKSPACE: return "JSSA_ERR_WORKSPACE";
    case JSSA_ERR_MISALIGNED: return "JSSA_ERR_MISALIGNED";
    case JSSA_ERR_HIP: return "JSSA_ERR_HIP";
    case JSSA_ERR_TOO_LARGE: return "JSSA_ERR_TOO_LARGE";
  }
  return "JSSA_ERR_UNKNOWN";
}

int32_t jssa_check_desc(const jssa_desc* desc, int32_t op) {
  if (op < 0 || op > JSSA_OP_VOTE) return JSSA_ERR_INVALID_ARG;
  return check(desc, op);
}

size_t jssa_workspace_bytes(const jssa_desc* desc, int32_t op) {
  if (!desc || op < JSSA_OP_TOPK || op > JSSA_OP_VOTE) return 0;
  Workspace w;
  if (!workspace_layout(*desc, op, &w)) return 0;
  return w.total;
}

int32_t jssa_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws && ws_bytes) return JSSA_ERR_INVALID_ARG;
  if (ws && (reinterpret_cast<uintptr_t>(ws) % 256) != 0) return JSSA_ERR_WORKSPACE;
  return to_status(launch_zero(ws, ws_bytes, as_stream(stream)));
}

int32_t jssa_workspace_status(void* ws, size_t ws_bytes, uint32_t* status_out, int32_t clear, void* stream) {
  if (!ws || !status_out) return JSSA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) % 256) != 0 || ws_bytes < kQueueWords * sizeof(uint32_t))
    return JSSA_ERR_WORKSPACE;
  if (!aligned16(status_out)) return JSSA_ERR_MISALIGNED;
  return to_status(launch_status(static_cast<uint32_t*>(ws), status_out, clear != 0, as_stream(stream)));
}

int32_t jssa_append_kv(const jssa_desc* desc, const void* k_new, const void* v_new, int32_t n_new,
                       const int32_t* pos, const float* P, void* k_cache, void* v_cache,
                       void* kp_cache, void* stream) {
  JSSA_TRY(check(desc, 0));
  if (n_new < 0) return JSSA_ERR_INVALID_ARG;
  if (!pos || !P || !k_cache || !kp_cache) return JSSA_ERR_INVALID_ARG;
  const bool mla = desc->layout == JSSA_LAYOUT_MLA;
  if (k_new && !mla && (!v_new || !v_cache)) return JSSA_ERR_INVALID_ARG;
  if (!aligned16(P) || !aligned16(k_cache) || !aligned16(kp_cache) || !aligned16(pos) ||
      (k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)) || (v_cache && !aligned16(v_cache)))
    return JSSA_ERR_MISALIGNED;
  if (n_new == 0) return JSSA_OK;
  return to_status(launch_append(*desc, k_new, v_new, n_new, pos, P, k_cache, v_cache, kp_cache,
                                 as_stream(stream)));
}

int32_t jssa_score(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                   const int32_t* seq_lens, float* scores, void* ws, size_t ws_bytes, void* stream) {
  JSSA_TRY(check(desc, JSSA_OP_SCORE));
  if (!q || !P || !kp_cache || !seq_lens || !scores) return JSSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(P) || !aligned16(kp_cache) || !aligned16(seq_lens) || !aligned16(scores))
    return JSSA_ERR_MISALIGNED;
  if (desc->layout == JSSA_LAYOUT_MLA) {
    Workspace lay;
    JSSA_TRY(check_ws(*desc, JSSA_OP_SCORE, ws, ws_bytes, &lay));
    char* base = static_cast<char*>(ws);
    hipError_t e = launch_mla_qproj(*desc, q, P, base, lay, as_stream(stream));
    if (e == hipSuccess) e = launch_mla_scan(*desc, kp_cache, seq_lens, scores, false, base, lay, as_stream(stream));
    return to_status(e);
  }
  Workspace none;
  return to_status(launch_score(*desc, q, P, kp_cache, seq_lens, scores, nullptr, none, as_stream(stream)));
}

int32_t jssa_topk(const jssa_desc* desc, const float* scores, const int32_t* seq_lens,
                  int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream) {
  JSSA_TRY(check(desc, JSSA_OP_TOPK));
  if (!scores || !seq_lens || !idx || !n_sel) return JSSA_ERR_INVALID_ARG;
  if (!aligned16(scores) || !aligned16(seq_lens) || !aligned16(idx) || !aligned16(n_sel))
    return JSSA_ERR_MISALIGNED;
  Workspace lay;
  JSSA_TRY(check_ws(*desc, JSSA_OP_TOPK, ws, ws_bytes, &lay));
  char* base = static_cast<char*>(ws);
  hipStream_t s = as_stream(stream);
  hipError_t e = launch_hist(*desc, scores, seq_lens, base, lay, s);
  if (e == hipSuccess) e = launch_candidates(*desc, scores, seq_lens, base, lay, s);
  if (e == hipSuccess)
    e = launch_resolve_attend(*desc, true, false, nullptr, nullptr, nullptr, idx, n_sel, seq_lens, nullptr,
                              nullptr, base, lay, s);
  return to_status(e);
}

int32_t jssa_indexed_attn(const jssa_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* idx, const int32_t* n_sel,
                          void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  JSSA_TRY(check(desc, JSSA_OP_ATTN));
  const bool mla = desc->layout == JSSA_LAYOUT_MLA;
  if (!q || !k_cache || (!mla && !v_cache) || !idx || !n_sel || !out) return JSSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(idx) ||
      !aligned16(n_sel) || !aligned16(out) || (lse && !aligned16(lse)))
    return JSSA_ERR_MISALIGNED;
  Workspace lay;
  JSSA_TRY(check_ws(*desc, JSSA_OP_ATTN, ws, ws_bytes, &lay));
  if (mla)
    return to_status(launch_mla_attend(*desc, q, k_cache, idx, n_sel, nullptr, out, lse, static_cast<char*>(ws),
                                       lay, as_stream(stream)));
  if (lay.pipe)
    return to_status(launch_pipe_attend(*desc, q, k_cache, v_cache, idx, n_sel, out, lse, static_cast<char*>(ws),
                                        lay, as_stream(stream)));
  return to_status(launch_resolve_attend(*desc, false, true, q, k_cache, v_cache, const_cast<int32_t*>(idx),
                                         const_cast<int32_t*>(n_sel), nullptr, out, lse,
                                         static_cast<char*>(ws), lay, as_stream(stream)));
}

int32_t jssa_reuse_step(const jssa_desc* desc, const void* k_new, const void* v_new,
                        const int32_t* pos, const void* q, void* k_cache, void* v_cache,
                        const int32_t* idx, const int32_t* n_sel, void* out, float* lse, void* ws,
                        size_t ws_bytes, void* stream) {
  JSSA_TRY(check(desc, JSSA_OP_DECODE));
  const bool mla = desc->layout == JSSA_LAYOUT_MLA;
  if (!q || !k_cache || (!mla && !v_cache) || !idx || !n_sel || !out) return JSSA_ERR_INVALID_ARG;
  if (k_new && (!pos || (!mla && !v_new))) return JSSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(idx) || !aligned16(n_sel) ||
      !aligned16(out) || (lse && !aligned16(lse)) || (k_new && (!aligned16(k_new) || !aligned16(pos))) ||
      (k_new && !mla && !aligned16(v_new)))
    return JSSA_ERR_MISALIGNED;
  Workspace lay;
  JSSA_TRY(check_ws(*desc, JSSA_OP_DECODE, ws, ws_bytes, &lay));
  char* base = static_cast<char*>(ws);
  hipStream_t s = as_stream(stream);
  if (k_new) {
    const hipError_t e = launch_copy_new(*desc, k_new, mla ? nullptr : v_new, pos, k_cache, v_cache, s);
    if (e != hipSuccess) return to_status(e);
  }
  if (mla)
    return to_status(launch_mla_attend(*desc, q, k_cache, idx, n_sel, nullptr, out, lse, base, lay, s));
  if (lay.pipe) return to_status(launch_pipe_attend(*desc, q, k_cache, v_cache, idx, n_sel, out, lse, base, lay, s));
  return to_status(launch_resolve_attend(*desc, false, true, q, k_cache, v_cache, const_cast<int32_t*>(idx),
                                         const_cast<int32_t*>(n_sel), nullptr, out, lse, base, lay, s));
}

}  // extern "C"

namespace jssa {

// Host-side checks of a decode's arguments (everything but the workspace).
int32_t check_decode_args(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                          const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                          float* lse, int32_t* idx_out, int32_t* n_sel_out, const NewToken* nt, void* const* ev) {
  JSSA_TRY(check(desc, JSSA_OP_DECODE));
  const bool mla = desc->layout == JSSA_LAYOUT_MLA;
  if (!q || !P || !kp_cache || !k_cache || (!mla && !v_cache) || !seq_lens || !out) return JSSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(P) || !aligned16(kp_cache) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(seq_lens) || !aligned16(out) || (lse && !aligned16(lse)) ||
      (idx_out && !aligned16(idx_out)) || (n_sel_out && !aligned16(n_sel_out)))
    return JSSA_ERR_MISALIGNED;
  if (ev)
    for (int i = 0; i < 4; ++i)
      if (!ev[i]) return JSSA_ERR_INVALID_ARG;
  if (nt) {  // the step's new token: rows and positions (GQA: the value row and cache too)
    if (!nt->k_new || !nt->pos || (!mla && (!nt->v_new || !nt->v_cache))) return JSSA_ERR_INVALID_ARG;
    if (!aligned16(nt->k_new) || !aligned16(nt->pos) || (!mla && !aligned16(nt->v_new))) return JSSA_ERR_MISALIGNED;
  }
  return JSSA_OK;
}

// The decode's launches on a workspace whose layout is `lay` (checked by the caller).
int32_t decode_launch(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                      const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out, float* lse,
                      int32_t* idx_out, int32_t* n_sel_out, char* base, const Workspace& lay, const NewToken* nt,
                      void* const* ev, void* stream) {
  const bool mla = desc->layout == JSSA_LAYOUT_MLA;
  float* scores = reinterpret_cast<float*>(base + lay.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + lay.idx);
  int32_t* n_sel = n_sel_out ? n_sel_out : reinterpret_cast<int32_t*>(base + lay.n_sel);
  hipStream_t s = as_stream(stream);
  if (lay.pipe)
    return to_status(launch_pipeline(*desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, idx, n_sel,
                                     base, lay, nt, ev, s));
  // MLA (MAX): the step's append and the query projection share the first launch
  const bool prep = mla && nt && mla_prep_fusable(*desc);
  if (nt && !prep) {  // the staged launches: the append is a launch of its own, first
    const hipError_t ea = launch_append(*desc, nt->k_new, nt->v_new, 1, nt->pos, P, nt->k_cache, nt->v_cache,
                                        nt->kp_cache, s);
    if (ea != hipSuccess) return to_status(ea);
  }
  auto mark = [&](int i) { return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess; };
  if (mla) {
    hipError_t e = prep ? launch_mla_prep(*desc, nt->k_new, nt->pos, P, nt->k_cache, nt->kp_cache, q, base, lay, s)
                        : launch_mla_qproj(*desc, q, P, base, lay, s);
    // events [0] and [1] take the score scan kernel's own start and end
    if (e == hipSuccess) e = launch_mla_scan(*desc, kp_cache, seq_lens, scores, true, base, lay, s, ev);
    if (e == hipSuccess) e = launch_candidates(*desc, scores, seq_lens, base, lay, s, true);
    if (e == hipSuccess) e = mark(2);
    if (e == hipSuccess) e = launch_select_rows(*desc, seq_lens, idx, n_sel, base, lay, s);
    if (e == hipSuccess) e = launch_mla_attend(*desc, q, k_cache, idx, n_sel, nullptr, out, lse, base, lay, s);
    if (e == hipSuccess) e = mark(3);
    return to_status(e);
  }
  hipError_t e = mark(0);
  if (e == hipSuccess) e = launch_score(*desc, q, P, kp_cache, seq_lens, scores, base, lay, s);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess) e = launch_candidates(*desc, scores, seq_lens, base, lay, s);
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess)
    e = launch_resolve_attend(*desc, true, true, q, k_cache, v_cache, idx, n_sel, seq_lens, out, lse, base,
                              lay, s);
  if (e == hipSuccess) e = mark(3);
  return to_status(e);
}

}  // namespace jssa

extern "C" {

static int32_t decode_impl(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                           const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                           void* out, float* lse, int32_t* idx_out, int32_t* n_sel_out,
                           void* ws, size_t ws_bytes, const NewToken* nt, void* const* ev, void* stream) {
  JSSA_TRY(check_decode_args(desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, idx_out, n_sel_out, nt,
                             ev));
  Workspace lay;
  JSSA_TRY(check_ws(*desc, JSSA_OP_DECODE, ws, ws_bytes, &lay));
  return decode_launch(desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, idx_out, n_sel_out,
                       static_cast<char*>(ws), lay, nt, ev, stream);
}

int32_t jssa_decode(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                    const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                    void* out, float* lse, int32_t* idx_out, int32_t* n_sel_out,
                    void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, idx_out, n_sel_out,
                     ws, ws_bytes, nullptr, nullptr, stream);
}

int32_t jssa_decode_profiled(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                             const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                             void* out, float* lse, int32_t* idx_out, int32_t* n_sel_out,
                             void* ws, size_t ws_bytes, void* const* stage_events, void* stream) {
  if (!stage_events) return JSSA_ERR_INVALID_ARG;
  return decode_impl(desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, idx_out, n_sel_out,
                     ws, ws_bytes, nullptr, stage_events, stream);
}

int32_t jssa_decode_step(const jssa_desc* desc, const void* k_new, const void* v_new, const int32_t* pos,
                         const void* q, const float* P, void* kp_cache, void* k_cache, void* v_cache,
                         const int32_t* seq_lens, void* out, float* lse, int32_t* idx_out,
                         int32_t* n_sel_out, void* ws, size_t ws_bytes, void* const* stage_events,
                         void* stream) {
  JSSA_TRY(check(desc, JSSA_OP_DECODE));
  const bool mla = desc->layout == JSSA_LAYOUT_MLA;
  const NewToken nt{k_new, mla ? nullptr : v_new, pos, k_cache, v_cache, kp_cache};
  return decode_impl(desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, idx_out, n_sel_out,
                     ws, ws_bytes, &nt, stage_events, stream);
}

int32_t jssa_vote_select(const jssa_desc* desc, const float* scores, const int32_t* seq_lens, int32_t* idx,
                         int32_t* n_sel, void* ws, size_t ws_bytes, void* stream) {
  JSSA_TRY(check(desc, JSSA_OP_VOTE));
  if (!scores || !seq_lens || !idx || !n_sel) return JSSA_ERR_INVALID_ARG;
  if (!aligned16(scores) || !aligned16(seq_lens) || !aligned16(idx) || !aligned16(n_sel))
    return JSSA_ERR_MISALIGNED;
  Workspace lay;
  JSSA_TRY(check_ws(*desc, JSSA_OP_VOTE, ws, ws_bytes, &lay));
  return to_status(launch_vote_select(*desc, scores, seq_lens, idx, n_sel, static_cast<char*>(ws), lay,
                                      as_stream(stream)));
}

int32_t jssa_gather_kv(const jssa_desc* desc, const void* k_cache, const void* v_cache, const int32_t* idx,
                       const int32_t* n_sel, void* k_packed, void* v_packed, int32_t* packed_lens,
                       void* stream) {
  JSSA_TRY(check(desc, JSSA_OP_ATTN));
  const bool mla = desc->layout == JSSA_LAYOUT_MLA;
  if (!k_cache || !idx || !n_sel || !k_packed || (!mla && (!v_cache || !v_packed))) return JSSA_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(idx) || !aligned16(n_sel) ||
      !aligned16(k_packed) || !aligned16(v_packed) || (packed_lens && !aligned16(packed_lens)))
    return JSSA_ERR_MISALIGNED;
  return to_status(launch_gather_kv(*desc, k_cache, v_cache, idx, n_sel, k_packed, v_packed, packed_lens,
                                    as_stream(stream)));
}

int32_t jssa_dense_decode(const jssa_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* seq_lens, void* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream) {
  JSSA_TRY(check(desc, JSSA_OP_DENSE));
  const bool mla = desc->layout == JSSA_LAYOUT_MLA;
  if (!q || !k_cache || (!mla && !v_cache) || !seq_lens || !out) return JSSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(seq_lens) ||
      !aligned16(out) || (lse && !aligned16(lse)))
    return JSSA_ERR_MISALIGNED;
  Workspace lay;
  JSSA_TRY(check_ws(*desc, JSSA_OP_DENSE, ws, ws_bytes, &lay));
  if (mla)
    return to_status(launch_mla_attend(*desc, q, k_cache, nullptr, nullptr, seq_lens, out, lse,
                                       static_cast<char*>(ws), lay, as_stream(stream)));
  if (lay.pipe)
    return to_status(launch_pipe_dense(*desc, q, k_cache, v_cache, seq_lens, out, lse, static_cast<char*>(ws), lay,
                                       as_stream(stream)));
  return to_status(launch_resolve_attend(*desc, false, true, q, k_cache, v_cache, nullptr, nullptr, seq_lens,
                                         out, lse, static_cast<char*>(ws), lay, as_stream(stream)));
}

}  // extern "C"
