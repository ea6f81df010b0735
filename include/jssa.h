/*
 * jssa.h — C ABI of the MI355X (gfx950) token-level sparse decode library.
 *
 * One decode step of Joint Subspace Sparse Attention, as described in
 * "Joint Subspace Sparse Attention for Efficient Long-Context Decoding"
 * (paperlayer.ai summary of arXiv 2610.19026v1; cited below as "JSSA
 * summary" with its section or figure):
 *
 *   1. every cached token is scored in a shared low-rank query-key subspace
 *      using a projected-key cache Kp = K P (Figure 1, sections 3.1, 3.2, 3.4);
 *   2. each (sequence, KV head) keeps its own top-k positions (Figure 1,
 *      section 1, appendix A.3, section E.3);
 *   3. the query heads of each KV head attend over those positions, reading
 *      the original full-dimensional K/V rows in place from the standard GQA
 *      cache, with no gather buffer and one launch for all heads (section 3.3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every array argument is a DEVICE pointer, allocated and owned by
 *   the caller.  The library never allocates or frees memory and keeps no
 *   state between calls.  The descriptor itself is a HOST pointer read during
 *   the call only.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Every call only enqueues work on it and returns without
 *   synchronising.
 * Errors: arguments are validated on the host before anything is enqueued;
 *   a failing check returns a negative jssa_status and enqueues nothing.  A
 *   failed kernel launch returns JSSA_ERR_HIP.  Values that live in device
 *   memory (seq_lens, pos) are not visible to the host: kernels clamp
 *   seq_lens[b] to [0, t_max] and skip appended rows beyond t_max.
 * Workspace: entry points that take `ws` need at least
 *   jssa_workspace_bytes(desc, op) bytes, 256-byte aligned, that were zeroed
 *   once (jssa_workspace_init) before first use.  Every call leaves the
 *   counters in the workspace zeroed again, so one workspace may be reused by
 *   calls serialised on one stream; concurrent calls need distinct workspaces.
 * Layouts (row-major, innermost last):
 *   q         [B, Hq, d_k]               dtype kv_dtype
 *   k_cache   [B, t_max, Hkv, d_k]       dtype kv_dtype
 *   v_cache   [B, t_max, Hkv, d_v]       dtype kv_dtype  (MLA: unused; V is
 *                                        the first d_v columns of each K row)
 *   P         [Hkv, d_k, rank]           float32, orthonormal columns
 *   kp_cache  [B, Hkv, t_max, rank]      dtype kp_dtype
 *   seq_lens  [B]                        int32, tokens cached per sequence
 *   scores    [B, Hkv, t_max]            float32
 *   idx       [B, Hkv, topk + window]    int32
 *   n_sel     [B, Hkv]                   int32
 *   out       [B, Hq, d_v]               dtype out_dtype
 *   lse       [B, Hq]                    float32 (natural log), may be NULL
 * Query head hq belongs to KV head hq / G, G = Hq / Hkv.  Every base pointer
 * must be 16-byte aligned.
 */
#ifndef JSSA_H
#define JSSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JSSA_ABI_VERSION 10

typedef enum {
  JSSA_OK = 0,
  JSSA_ERR_INVALID_ARG = -1,  /* null pointer, inconsistent sizes, bad enum */
  JSSA_ERR_UNSUPPORTED = -2,  /* valid but not built: shape/dtype combination */
  JSSA_ERR_WORKSPACE = -3,    /* workspace missing, too small or misaligned */
  JSSA_ERR_MISALIGNED = -4,   /* a data pointer is not 16-byte aligned */
  JSSA_ERR_HIP = -5,          /* a HIP launch failed */
  JSSA_ERR_TOO_LARGE = -6     /* the call needs more than the static scratch of
                                 jssa_decode_step_static */
} jssa_status;

/* JSSA_FP8_E4M3 (the OCP 8-bit format E4M3: bias 7, largest value 448, no
 * infinity) is a projected-key cache dtype only (JSSA summary appendix A.3:
 * the scoring cache is FP8; section E.2: it halves that cache against bf16).
 * Codes are stored one byte per element, scale-free; the projection rounds to
 * nearest even and saturates at +-448.  Built for GQA with bf16 q/K/V and
 * rank 32 or 64. */
typedef enum { JSSA_F32 = 0, JSSA_BF16 = 1, JSSA_FP8_E4M3 = 2 } jssa_dtype;

/* How a KV head reduces the subspace scores of its G query heads.
 * MAX: s_t = max_g (q_g P).Kp_t.  MEAN: s_t = mean_g (q_g P).Kp_t, which is
 * the JSSA summary's group-mean query (Figure 1, sections 3.1 and 3.2). */
typedef enum { JSSA_REDUCE_MAX = 0, JSSA_REDUCE_MEAN = 1 } jssa_reduce;

/* GQA: standard [B, T, Hkv, d] K and V caches.  MLA: one shared latent row
 * per token (Hkv = 1); the value is the first d_v columns of that row and
 * selection yields one index set per sequence (JSSA summary section 3.3).
 * MLA builds: d_k = 576, d_v = 512, rank 32 or 64, Hq = 64 or 128, bf16 q,
 * K and Kp; both contractions of scoring and attention run on the matrix
 * cores.  v_cache is unused and may be NULL. */
typedef enum { JSSA_LAYOUT_GQA = 0, JSSA_LAYOUT_MLA = 1 } jssa_layout;

typedef enum {
  JSSA_OP_TOPK = 1,    /* jssa_topk */
  JSSA_OP_ATTN = 2,    /* jssa_indexed_attn */
  JSSA_OP_DECODE = 3,  /* jssa_decode */
  JSSA_OP_DENSE = 4,   /* jssa_dense_decode */
  JSSA_OP_SCORE = 5,   /* jssa_score */
  JSSA_OP_VOTE = 6     /* jssa_vote_select */
} jssa_op;

typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t n_q_heads;   /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;  /* Hkv */
  int32_t d_k;         /* query/key head dim (GQA: 64 or 128; MLA: 576) */
  int32_t d_v;         /* value head dim (GQA: == d_k; MLA: 512) */
  int32_t rank;        /* scoring rank r (16, 32 or 64) */
  int32_t t_max;       /* cache capacity in tokens, 1 .. 2^24 */
  int32_t topk;        /* budget k >= 0 */
  int32_t window;      /* W >= 0 trailing tokens always attended; k + W >= 1 */
  int32_t kv_dtype;    /* jssa_dtype of q, K and V */
  int32_t kp_dtype;    /* jssa_dtype of the projected-key cache */
  int32_t out_dtype;   /* jssa_dtype of the attention output */
  int32_t reduce;      /* jssa_reduce */
  int32_t layout;      /* jssa_layout */
  float scale;         /* softmax scale applied to q.K, e.g. 1/sqrt(d_k) */
} jssa_desc;

/* Version of this ABI (JSSA_ABI_VERSION). */
int32_t jssa_abi_version(void);

/* Static, human-readable name of a status code. */
const char* jssa_status_str(int32_t status);

/* Checks a descriptor without touching the GPU: JSSA_OK if the library can
 * run `op` (a jssa_op, or 0 for the append/score entry points) for it. */
int32_t jssa_check_desc(const jssa_desc* desc, int32_t op);

/* Bytes of workspace `op` needs for `desc` (0 if the descriptor is invalid). */
size_t jssa_workspace_bytes(const jssa_desc* desc, int32_t op);

/* Zero-fills a workspace (a fill kernel on `stream`, safe inside graph
 * capture).  Needed once before a workspace's first use. */
int32_t jssa_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Device-side diagnostics of a workspace.  Entry points that take `ws`
 * record, in its first 256 bytes, sticky words that accumulate over calls
 * until cleared.  This enqueues on `stream` a copy of JSSA_STATUS_WORDS
 * uint32 words into status_out (a DEVICE array, 16-byte aligned) and, if
 * `clear` is nonzero, resets them to zero; it does not synchronise (read
 * status_out after the stream has reached this point).
 *   status_out[JSSA_STATUS_WAIT_TIMEOUT]  nonzero if a bounded in-kernel wait
 *       gave up (a workgroup waited seconds for a value another workgroup of
 *       the same launch publishes).  It means a broken invariant, never a
 *       normal outcome: the selections and outputs of the calls since the last
 *       clear must be treated as wrong.
 *   status_out[JSSA_STATUS_EXACT_REDO]    rows re-selected exactly because the
 *       sampled threshold of the fused decode admitted fewer than k tokens
 *       (results stay exact; a count only).
 *   status_out[JSSA_STATUS_RANGE_SPLIT]   fused decode scans whose rows'
 *       tiles were split into equal contiguous ranges across rows instead of
 *       per row: fewer score workgroups than rows, or rows of unequal lengths
 *       whose per-row split would leave some runs more than a tile longer
 *       than the even share (a count only).
 *   status_out[JSSA_STATUS_GLOBAL_CUT]    rows of the fused decode whose
 *       candidates exceeded shared memory, so that the exact cut ran over
 *       global memory (a count only).
 * ws: a workspace of any op (at least 256 bytes, 256-byte aligned).
 * Calls that use the workspace concurrently race with the copy and clear. */
#define JSSA_STATUS_WORDS 4
#define JSSA_STATUS_WAIT_TIMEOUT 0
#define JSSA_STATUS_EXACT_REDO 1
#define JSSA_STATUS_RANGE_SPLIT 2
#define JSSA_STATUS_GLOBAL_CUT 3
int32_t jssa_workspace_status(void* ws, size_t ws_bytes, uint32_t* status_out, int32_t clear,
                              void* stream);

/* Append and project (JSSA summary section E.1: each newly generated key is
 * projected into the scoring cache; sections 3.1 and 3.4: the cache holds
 * Kp = K P per KV head and is used only for scoring).
 * For b < B and j < n_new, with t = pos[b] + j (rows with t >= t_max are
 * skipped):
 *   k_cache[b,t,h,:] = k_new[b,j,h,:]; v_cache[b,t,h,:] = v_new[b,j,h,:]
 *   kp_cache[b,h,t,i] = round(sum_d k_cache[b,t,h,d] * P[h,d,i])
 * accumulated in fp32 and rounded to kp_dtype (bf16: nearest-even).
 * k_new/v_new are [B, n_new, Hkv, d] (GQA) or [B, n_new, 1, d_k] (MLA, no v).
 * If k_new is NULL the rows are already in the cache and only the projection
 * is done (bulk prefill of the scoring cache); v_new is then ignored.
 * pos: int32 [B] device array of first positions. */
int32_t jssa_append_kv(const jssa_desc* desc, const void* k_new, const void* v_new, int32_t n_new,
                       const int32_t* pos, const float* P, void* k_cache, void* v_cache,
                       void* kp_cache, void* stream);

/* Subspace scores (JSSA summary Figure 1 and section 3.1): for every
 * candidate t < seq_lens[b] - window,
 *   scores[b,h,t] = reduce_g sum_i (q[b,h*G+g,:] P[h])[i] * kp_cache[b,h,t,i]
 * with the projected query kept in fp32.  Entries t >= seq_lens[b] - window
 * are not written.  MLA: the projected queries are fp32 and enter the
 * matrix-core product as two bf16 terms (hi = nearest bf16, lo = nearest
 * bf16 of the remainder), so |error| <= 2^-17 * sum_i |qp_i Kp_i| per head;
 * MEAN projects the mean of the Hq queries.
 * Workspace op JSSA_OP_SCORE: MLA descriptors need it (the projected-query
 * fragments); GQA descriptors do not use it and may pass NULL. */
int32_t jssa_score(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                   const int32_t* seq_lens, float* scores, void* ws, size_t ws_bytes, void* stream);

/* Per-(sequence, KV head) selection (JSSA summary Figure 1, section 3.1,
 * appendix A.3): among the candidates t < T_b - W (T_b = seq_lens[b]) keep
 * the min(k, T_b - W) largest scores, ties to the lower index, NaN below every
 * number, -0.0 equal to +0.0; then append the window T_b-W .. T_b-1.
 * idx[b,h,:] lists the selected candidates in ascending order followed by the
 * window; n_sel[b,h] = min(k, max(T_b-W,0)) + min(W, T_b).  Entries past
 * n_sel are not written.  Exact: the result is a function of the fp32 score
 * bits only.  Workspace op JSSA_OP_TOPK. */
int32_t jssa_topk(const jssa_desc* desc, const float* scores, const int32_t* seq_lens,
                  int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream);

/* Gather-free indexed attention (JSSA summary section 3.3): for each query
 * head hq (KV head h = hq / G) over the n_sel[b,h] tokens idx[b,h,:],
 *   out[b,hq,:] = sum_t softmax_t(scale * q[b,hq].K[b,t,h]) V[b,t,h,:]
 *   lse[b,hq]   = log sum_t exp(scale * q[b,hq].K[b,t,h])
 * reading each selected K/V row in place once for all G query heads; fp32
 * accumulation; index chunks merged by a log-sum-exp combine.  n_sel = 0
 * gives out = 0 and lse = -inf.  Indices should lie in [0, t_max); others are
 * clamped into that range.  MLA: all Hq heads share the one index set per
 * sequence; the value is the first d_v columns of the selected row; q.K and
 * P V run on the matrix cores with fp32 accumulation and the probabilities
 * entered as bf16 hi + lo terms (about 16 significant bits).  Shapes with a
 * fused decode build run the decode's own attention over parts of each list
 * and its in-launch merge of the parts (the same results as the attention
 * inside jssa_decode).
 * Workspace op JSSA_OP_ATTN. */
int32_t jssa_indexed_attn(const jssa_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* idx, const int32_t* n_sel,
                          void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* One sparse decode step: the result of jssa_score -> jssa_topk ->
 * jssa_indexed_attn (JSSA summary Figure 1 and section E.1), bit-identical in
 * idx / n_sel, with intermediates in the workspace.  For the shapes with a
 * fused build (bf16: d 128 rank 32 G 4, d 128 rank 64 G 1, d 64 rank 16 G 4;
 * bf16 K/V with FP8 projected keys: d 128 rank 32 G 4, d 128 rank 64 G 1;
 * f32: d 64 rank 16 G 4, d 128 rank 32 G 2; GQA layout; topk + window at most
 * 32768) it runs in two launches: a scan that scores every candidate and
 * keeps, per tile, the tokens at or above a threshold taken from a strided
 * sample of the row's scores; then a few workgroups per (sequence, KV head)
 * that each select the row exactly among those tokens (re-selecting it exactly
 * in the rare case fewer than k passed the threshold), keep their part of the
 * list, attend over it, and merge the parts (the row's last part).  The
 * attention over a part is the one jssa_indexed_attn runs on these shapes, so
 * both give the same outputs for the same lists.  Other shapes run the
 * stand-alone kernels in sequence (MLA: query projection, score scan with the
 * first-digit histogram, candidate pass, the exact selection of each row by
 * one workgroup, attention, chunk merge).
 * idx_out / n_sel_out may be NULL; when given they receive the selection.
 * The new token is expected to be appended (jssa_append_kv) before this
 * call.  Workspace op JSSA_OP_DECODE. */
int32_t jssa_decode(const jssa_desc* desc, const void* q, const float* P, const void* kp_cache,
                    const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                    void* out, float* lse, int32_t* idx_out, int32_t* n_sel_out,
                    void* ws, size_t ws_bytes, void* stream);

/* jssa_decode that also records four caller-created HIP events
 * (stage_events[i] is a hipEvent_t created with timing; the array is a host
 * array) on `stream`, around its launches -- the per-component latency
 * breakdown of JSSA summary section E.1 (scan, selection, attention).  Fused
 * build: [0] and [1] are the scan kernel's own start and end (the kernel's
 * execution, as a profiler reports it; the scan also writes the candidates),
 * [2] is recorded after the select/attend launch (selection, attention and
 * merge), [3] right after [2].  Other GQA shapes: [0] before the score scan,
 * [1] after it, [2] after the candidate pass, [3] after the resolve +
 * attention.  MLA: [0] and [1] the score scan kernel's start and end, [2]
 * after the candidate pass, [3] after the selection, the attention and the
 * chunk merge. */
int32_t jssa_decode_profiled(const jssa_desc* desc, const void* q, const float* P,
                             const void* kp_cache, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, void* out, float* lse, int32_t* idx_out,
                             int32_t* n_sel_out, void* ws, size_t ws_bytes,
                             void* const* stage_events, void* stream);

/* One whole decode step: jssa_append_kv of one new token per sequence
 * (n_new = 1: k_new[b,0,h,:] / v_new[b,0,h,:] written at t = pos[b] and the
 * key projected into kp_cache) followed by jssa_decode on the updated caches
 * (JSSA summary section E.1: the new key is projected when it is generated,
 * then the step scores, selects and attends).  Results are bit-identical to
 * the two calls in sequence.  In the fused build the append runs inside the
 * scan launch: each (sequence, KV head) row's sample first publishes the
 * row's threshold, then writes the new K/V rows and the projected key and
 * marks the row as appended; the score run whose range holds pos[b] waits for
 * that mark and re-scores the one step that holds pos[b] from the stored row;
 * no launch of its own.  Other shapes launch the append first, before
 * stage_events[0] (the MLA layout with the MAX reduction in one launch with
 * the query projection).  k_new / v_new: [B, 1, Hkv, d] (MLA: [B, 1, 1, d_k], v_new
 * and v_cache unused, may be NULL); pos: int32 [B] device array; positions
 * outside [0, t_max) are not written.  The caches are read and written in
 * place.  stage_events may be NULL, else as for jssa_decode_profiled.
 * Workspace op JSSA_OP_DECODE. */
int32_t jssa_decode_step(const jssa_desc* desc, const void* k_new, const void* v_new,
                         const int32_t* pos, const void* q, const float* P, void* kp_cache,
                         void* k_cache, void* v_cache, const int32_t* seq_lens, void* out,
                         float* lse, int32_t* idx_out, int32_t* n_sel_out, void* ws,
                         size_t ws_bytes, void* const* stage_events, void* stream);

/* jssa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The intermediates live in one static
 * device array of JSSA_STATIC_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends; nothing is allocated or freed
 * by the call.  Same arguments (stage events excepted) and results, bit for
 * bit, as jssa_decode_step with a zeroed workspace.
 * Limits: the shapes with a fused decode build (GQA; see jssa_decode) only,
 * else JSSA_ERR_UNSUPPORTED; at most JSSA_STATIC_SCRATCH_ROWS (sequence, KV
 * head) rows, and jssa_workspace_bytes(desc, JSSA_OP_DECODE) plus the rows'
 * reserved state must fit the array, else JSSA_ERR_TOO_LARGE (for example
 * batch 16, 8 KV heads and t_max 131072 fit; the candidate slots take
 * 8 bytes per cached token and KV head).  The first call on a GPU enqueues
 * a zero fill of the array's counters on `stream`.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other host threads) race and give wrong results;
 * serialise them.  No workspace diagnostics are reported. */
#define JSSA_STATIC_SCRATCH_BYTES (160u << 20)
#define JSSA_STATIC_SCRATCH_ROWS 8192
int32_t jssa_decode_step_static(const jssa_desc* desc, const void* k_new, const void* v_new,
                                const int32_t* pos, const void* q, const float* P, void* kp_cache,
                                void* k_cache, void* v_cache, const int32_t* seq_lens, void* out,
                                float* lse, int32_t* idx_out, int32_t* n_sel_out, void* stream);

/* One decode step of a layer that reuses another layer's selection (JSSA
 * summary appendix C: with a model's own sparse-attention schedule, tokens
 * are selected only at indexer layers and the adjacent layers reuse those
 * indices).  Such a layer keeps no scoring cache: the step writes the new
 * token's K and V rows (k_new[b,0,h,:] / v_new[b,0,h,:] at t = pos[b], no
 * projection; positions outside [0, t_max) are not written; k_new == NULL:
 * nothing is appended), then attends over idx / n_sel exactly as
 * jssa_indexed_attn does.  idx / n_sel are an indexer layer's lists of the
 * same step ([B, Hkv, topk + window] and [B, Hkv], e.g. idx_out / n_sel_out of
 * its jssa_decode_step); both layers index the same token positions.  The
 * fused build runs the decode's own attention and merge of its parts; other
 * shapes the stand-alone attention.  MLA: k_new [B, 1, 1, d_k], v_new and
 * v_cache unused (may be NULL).  Workspace op JSSA_OP_DECODE. */
int32_t jssa_reuse_step(const jssa_desc* desc, const void* k_new, const void* v_new,
                        const int32_t* pos, const void* q, void* k_cache, void* v_cache,
                        const int32_t* idx, const int32_t* n_sel, void* out, float* lse, void* ws,
                        size_t ws_bytes, void* stream);

/* Head-shared soft-voting selection, the alternative the pages compare the
 * per-KV-head sets with (JSSA summary section E.3: one token set per
 * sequence).  The pages do not define the vote; here each KV head votes with
 * the softmax of its scaled scores over the sequence's candidates
 * t < T_b - W (scale = desc->scale; NaN scores get no vote), the votes are
 * summed over the KV heads,
 *   vote[b,t] = sum_h exp(scale s[b,h,t]) / sum_u exp(scale s[b,h,u]),
 * the top-k of the vote (as jssa_topk: ties to the lower index, then the
 * window) is taken once per sequence and written to every KV head's list:
 * idx[b,h,:] and n_sel[b,h] are the same for all h, in jssa_topk's format, so
 * jssa_indexed_attn attends over them unchanged.  scores: [B, Hkv, t_max]
 * fp32 (e.g. from jssa_score).  GQA layout, Hkv <= 64.  Workspace op
 * JSSA_OP_VOTE. */
int32_t jssa_vote_select(const jssa_desc* desc, const float* scores, const int32_t* seq_lens,
                         int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream);

/* Gather of the selected rows into packed buffers: the first half of the
 * gather-then-attend baseline that gather-free execution is compared against
 * (JSSA summary section 2.2 and Figure 2(b); section 4.7: with the same
 * selected tokens, gather-free execution roughly doubles the attention-stage
 * speedup).  For i < n_sel[b,h] (S = topk + window):
 *   k_packed[b,i,h,:] = k_cache[b, idx[b,h,i], h, :]   (v likewise)
 * with indices clamped into [0, t_max) as the attention clamps them; entries
 * i >= n_sel are not written.  The packed buffers [B, S, Hkv, d] keep the
 * cache layout, so jssa_dense_decode with t_max = S and seq_lens =
 * packed_lens attends over exactly the selected rows.  packed_lens (int32
 * [B], may be NULL) receives n_sel[b, 0].  MLA: one index list per sequence
 * (Hkv = 1), whole latent rows packed, v_cache / v_packed unused (may be
 * NULL).  No workspace. */
int32_t jssa_gather_kv(const jssa_desc* desc, const void* k_cache, const void* v_cache,
                       const int32_t* idx, const int32_t* n_sel, void* k_packed, void* v_packed,
                       int32_t* packed_lens, void* stream);

/* Full-KV decode attention over all t < seq_lens[b] (the comparison path of
 * JSSA summary section 4.5), same outputs as jssa_indexed_attn.
 * Workspace op JSSA_OP_DENSE. */
int32_t jssa_dense_decode(const jssa_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* seq_lens, void* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* JSSA_H */
