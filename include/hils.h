/*
 * libhils — HiLS (Hierarchical Landmark Sparse) attention on AMD Instinct
 * MI355X (gfx950).  C ABI.
 *
 * The operator (sources: "Hierarchical Sparse Attention Done Right",
 * abstract on the chatpaper page; ai-feeds summary, section "Method" >
 * "Input & chunking" and "Key modules" items 1-3; paper.oopus.info review,
 * sections 2-3):
 *   the sequence is cut into chunks of C = 64 tokens, each with one landmark
 *   key; query t scores every completed past chunk j < t/C through its
 *   landmark, s_tj = scale * <q_t, Klm_j>; it keeps the top-k of them (ties to
 *   the lower chunk index) plus its own chunk c = t/C (scored by Klm_c, not
 *   counted in k, attended causally); it runs softmax attention inside each
 *   kept chunk, o_tj; and returns o_t = sum_j w_tj o_tj with w the softmax of
 *   the kept chunks' scores.  scale is 1/sqrt(d) unless the caller passes
 *   another positive value.
 *
 * Common conventions
 *   Layouts are row-major with the head dim innermost:
 *     Q, K, V, O, dO     [B][H][L][d]
 *     K_lm               [B][H][N][d]        N = L / C
 *     idx                [B][H][L][k+1] int32: slots 0..m-1 hold the kept past
 *                        chunks in selection order (score desc, index asc),
 *                        m = min(k, t/C); slots m..k-1 hold -1; slot k holds t/C.
 *     sel_score, w, lse  [B][H][L][k+1] float: the fp32 chunk score, fusion
 *                        weight and chunk log-partition function of each slot
 *                        (-inf, 0, unspecified on unused slots).
 *   Element type (dt): HILS_BF16 (storage of Q,K,V,K_lm,O,dO as bf16) or
 *   HILS_FP32.  Arithmetic: products on MFMA with fp32 accumulation (bf16
 *   MFMA for bf16 inputs, fp32 MFMA for fp32 inputs); the per-pair partial
 *   outputs of the forward travel through the workspace as bf16 for both.
 *   Sizes: B, H >= 1; d in {64, 128}; C == 64; L a positive multiple of C;
 *   N = L/C <= 16384; 1 <= k <= 16; B*H*L*(k+1) < 2^31.
 *   Pointers are device pointers, 16-byte aligned, non-overlapping between
 *   inputs and outputs.  The caller allocates and frees every buffer,
 *   including the workspace (see hils_workspace_size); the library never
 *   allocates device memory and keeps no device state between calls.
 *   Every call validates all arguments on the host before touching the
 *   device, enqueues its kernels on `stream` (a hipStream_t, NULL = default
 *   stream) and returns without synchronising; outputs are valid once the
 *   stream has reached that point.  Faults inside a kernel surface at the
 *   caller's next synchronisation.  NaN/Inf inputs are not checked; the
 *   selection they produce is unspecified.  Calls on distinct streams with
 *   distinct buffers may run concurrently.
 *   Errors: a non-zero hils_status; hils_last_error() then returns a message
 *   (per calling thread) describing it.
 */
#ifndef HILS_H
#define HILS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HILS_OK = 0,
  HILS_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer */
  HILS_ERR_UNSUPPORTED = 2, /* valid but not implemented (d, C, k, dtype limits) */
  HILS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than hils_workspace_size */
  HILS_ERR_HIP = 4          /* the HIP runtime reported an error */
} hils_status;

typedef enum { HILS_BF16 = 0, HILS_FP32 = 1 } hils_dtype;

/* operation codes for hils_workspace_size */
enum {
  HILS_OP_SCORES = 0,
  HILS_OP_TOPK = 1,
  HILS_OP_FWD = 2,
  HILS_OP_DECODE = 3,
  HILS_OP_BWD = 4,
  HILS_OP_FWD_ML = 5
};

/* Message of the last non-OK status returned to the calling thread ("" if none). */
const char* hils_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int hils_version(void);

/*
 * OR into the operation code of hils_workspace_size when the call's inputs
 * are HILS_FP32: the forward's per-pair chunk outputs and the backward's
 * per-pair dQ parts are then kept in fp32 (bf16 for 16-bit inputs), so
 * HILS_OP_FWD, HILS_OP_FWD_ML and HILS_OP_BWD need more workspace.
 */
#define HILS_WS_FP32 256

/*
 * Bytes of workspace the operation needs for these sizes (0 if none; a
 * null workspace pointer is then accepted).  For HILS_OP_DECODE pass the
 * cache capacity L_max as L.  op may carry HILS_WS_FP32 (see above).
 * Returns 0 and sets hils_last_error for invalid sizes.
 */
size_t hils_workspace_size(int op, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk);

/*
 * Dense causal landmark scores (first step of the method: ai-feeds summary
 * "Key modules" item 1; oopus review section 2).
 *   S[b][h][t][j] = scale * <Q[b][h][t], K_lm[b][h][j]>  for j <= t/C,
 *                   -inf                                 for j >  t/C.
 * S: [B][H][L][N] float, written in full.  Materialises B*H*L*N floats:
 * meant for inspection and tests; the forward never forms this matrix.
 */
hils_status hils_landmark_scores(const void* Q, const void* K_lm, float* S, int64_t B, int64_t H, int64_t L,
                                 int64_t d, int64_t C, float scale, hils_dtype dt, void* stream);

/*
 * Causal top-k chunk selection fused with the scoring (ai-feeds summary
 * "Key modules" items 1-2: scores, top-k chunks, chunk-level softmax).
 * Writes idx, sel_score and (if w is non-null) the fusion weights w for every
 * query row.  Scores are never materialised.  Workspace:
 * hils_workspace_size(HILS_OP_TOPK, ...) bytes (16-byte aligned; the bf16
 * path keeps a copy of K_lm there, rows in MFMA fragment order), owned by
 * the caller and free again when the stream has run the call.
 */
hils_status hils_topk_select(const void* Q, const void* K_lm, int32_t* idx, float* sel_score, float* w,
                             int64_t B, int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk, float scale,
                             hils_dtype dt, void* ws, size_t ws_bytes, void* stream);

/*
 * Forward of the operator (whole method: abstract on the chatpaper page;
 * ai-feeds summary "Key modules" items 1-3).
 *   select = 1: compute the selection and write idx and sel_score;
 *   select = 0: read the caller's idx (same layout; slot k must hold t/C,
 *               past slots must be distinct chunks < t/C or -1, and the
 *               valid ones must come first) and write sel_score for it.
 * O (element type dt) is written for every row.  w_out and lse_out
 * ([B][H][L][k+1] float) are optional (null = not returned); the backward
 * pass needs both.  Workspace: hils_workspace_size(HILS_OP_FWD, ...).
 */
hils_status hils_sparse_attn_fwd(const void* Q, const void* K, const void* V, const void* K_lm, int32_t* idx,
                                 float* sel_score, int select, void* O, float* w_out, float* lse_out, int64_t B,
                                 int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk, float scale,
                                 hils_dtype dt, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step (the per-step landmark scan the ai-feeds summary names
 * under "Limitations"; the same operator for a single new query per head).
 *   q, k_new, v_new : [B][H][d] (element type dt)
 *   K_cache, V_cache: [B][H][L_max][d]; row n_ctx receives k_new / v_new
 *   K_lm_cache      : [B][H][N_max][d], N_max = ceil(L_max / C); the caller
 *                     must have written row n_ctx / C (the open chunk's
 *                     landmark) before the call.
 * The query at position n_ctx attends over keys 0..n_ctx:  past chunks
 * j < n_ctx/C are candidates, the open chunk n_ctx/C is its own chunk.
 * Outputs: o [B][H][d] (dt), idx and w [B][H][k+1] (as in the prefill layout).
 * 0 <= n_ctx < L_max.  Re-issuing a step with the same n_ctx is idempotent.
 * Workspace: hils_workspace_size(HILS_OP_DECODE, B, H, L_max, d, C, topk).
 */
hils_status hils_decode_step(const void* q, const void* k_new, const void* v_new, void* K_cache, void* V_cache,
                             const void* K_lm_cache, int64_t n_ctx, int64_t L_max, void* o, int32_t* idx, float* w,
                             int64_t B, int64_t H, int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Backward with the selection held fixed (native sparse training: ai-feeds
 * summary "Key modules" item 3 and "Output & training"; the retrieval
 * scores receive gradients through the fusion weights, abstract on the
 * chatpaper page).  Inputs: the forward's Q, K, V, K_lm (dt), the upstream
 * gradient dO (dt), and the forward's idx, w and lse.  Outputs (float,
 * written in full):  dQ, dK, dV [B][H][L][d];  dK_lm [B][H][N][d].
 * The gradient of the fusion weights uses D = sum_j w_j dO.o_j formed from
 * the per-chunk outputs, so the forward output O is not an input.
 * Workspace: hils_workspace_size(HILS_OP_BWD, ...).
 */
hils_status hils_sparse_attn_bwd(const void* Q, const void* K, const void* V, const void* K_lm, const void* dO,
                                 const int32_t* idx, const float* w, const float* lse, float* dQ, float* dK,
                                 float* dV, float* dK_lm, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
                                 int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes, void* stream);

/*
 * Separate retrieval queries (the low-rank query calibration that the
 * ai-feeds summary names under "Method" > "Input & chunking": an affine map
 * of Q, made by the caller, that serves the chunk retrieval).  Q_ret / q_ret
 * has Q's / q's layout and element type; it replaces Q in the landmark
 * scores, so in the selection and in the fusion weights, while the per-chunk
 * attention keeps Q.  A null Q_ret / q_ret is the plain entry point.
 *   hils_sparse_attn_fwd_rq : as hils_sparse_attn_fwd; with select = 0 the
 *                             caller's idx is scored with Q_ret.
 *   hils_decode_step_rq     : as hils_decode_step.
 *   hils_sparse_attn_bwd_rq : as hils_sparse_attn_bwd; dQ_ret [B][H][L][d]
 *                             float receives the score-path gradient
 *                             (sum_j ds_tj scale K_lm_j) and dQ the in-chunk
 *                             attention terms only; dK_lm sums ds_tj Q_ret_t.
 *                             Q_ret and dQ_ret are given together or both
 *                             null (else HILS_ERR_INVALID_ARG).
 * Workspaces are those of the plain entry points.  Pointers: 16-byte aligned.
 */
hils_status hils_sparse_attn_fwd_rq(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    int32_t* idx, float* sel_score, int select, void* O, float* w_out,
                                    float* lse_out, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
                                    int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                    void* stream);
hils_status hils_decode_step_rq(const void* q, const void* q_ret, const void* k_new, const void* v_new,
                                void* K_cache, void* V_cache, const void* K_lm_cache, int64_t n_ctx, int64_t L_max,
                                void* o, int32_t* idx, float* w, int64_t B, int64_t H, int64_t d, int64_t C,
                                int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes, void* stream);
hils_status hils_sparse_attn_bwd_rq(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ,
                                    float* dQ_ret, float* dK, float* dV, float* dK_lm, int64_t B, int64_t H,
                                    int64_t L, int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * Landmark-free chunks (the landmark-free alternative the ai-feeds summary
 * mentions under "Method" > "Input & chunking"): a chunk's landmark key is
 * the mean of its C keys (fp32 sum, rounded to the element type); for the
 * query's own chunk only the keys up to the query are averaged, so no key
 * after the query enters its scores.
 *   hils_chunk_means       : rows 0..n_chunks-1 of K_lm [B][H][N_lm][d] (dt)
 *                            = means of the key rows of each chunk of K
 *                            [B][H][L_k][d] (dt).  n_chunks*C <= L_k,
 *                            n_chunks <= N_lm.  Use it to fill the landmark
 *                            rows of the complete chunks of a decode cache.
 *   hils_sparse_attn_fwd_lf: as hils_sparse_attn_fwd_rq (Q_ret may be null),
 *                            but the landmarks are formed here: K_lm_out
 *                            [B][H][N][d] (dt, caller-owned) receives the key
 *                            means, which score the past chunks; the own
 *                            slot's sel_score and all fusion weights use the
 *                            causal mean of the own chunk.  Same workspace.
 *   hils_decode_step_lf    : as hils_decode_step_rq (q_ret may be null); the
 *                            step writes landmark row n_ctx/C of K_lm_cache
 *                            (the mean of keys C*(n_ctx/C) .. n_ctx, k_new
 *                            included) before reading it; rows of earlier
 *                            chunks must hold their key means (from
 *                            hils_chunk_means or from earlier steps).
 *   hils_sparse_attn_bwd_lf: as hils_sparse_attn_bwd_rq for the forward
 *                            above: K_lm is that forward's K_lm_out; dK also
 *                            carries the landmark paths (each past chunk's
 *                            mean gradient / C to its keys, and the own
 *                            slot's gradient to the keys it averaged, the
 *                            rounding of the means passed straight through);
 *                            dK_lm [B][H][N][d] float receives the past
 *                            chunks' mean gradient (already inside dK).
 */
hils_status hils_chunk_means(const void* K, void* K_lm, int64_t B, int64_t H, int64_t L_k, int64_t N_lm,
                             int64_t n_chunks, int64_t d, int64_t C, hils_dtype dt, void* stream);
hils_status hils_sparse_attn_fwd_lf(const void* Q, const void* Q_ret, const void* K, const void* V, void* K_lm_out,
                                    int32_t* idx, float* sel_score, int select, void* O, float* w_out,
                                    float* lse_out, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
                                    int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                    void* stream);
hils_status hils_sparse_attn_bwd_lf(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ,
                                    float* dQ_ret, float* dK, float* dV, float* dK_lm, int64_t B, int64_t H,
                                    int64_t L, int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt,
                                    void* ws, size_t ws_bytes, void* stream);
hils_status hils_decode_step_lf(const void* q, const void* q_ret, const void* k_new, const void* v_new,
                                void* K_cache, void* V_cache, void* K_lm_cache, int64_t n_ctx, int64_t L_max,
                                void* o, int32_t* idx, float* w, int64_t B, int64_t H, int64_t d, int64_t C,
                                int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes, void* stream);

/*
 * Several landmarks per chunk (ai-feeds summary, "Method" > "Input &
 * chunking": a few landmarks per chunk, usually its first and last token;
 * "Key modules" item 1: a softmax over a chunk's landmark scores before the
 * chunk-level one).  K_lm is [B][H][N][m][d] (dt), 1 <= m <= 16; the chunk
 * score is the log-sum-exp of its m landmark scores, for the past chunks and
 * the own chunk alike; with m = 1 it is the plain score.  Otherwise as
 * hils_sparse_attn_fwd_rq (Q_ret may be null).  No chunk score matrix is
 * formed; workspace: hils_workspace_size(HILS_OP_FWD_ML, ...) bytes, the same
 * as HILS_OP_FWD.
 */
hils_status hils_sparse_attn_fwd_ml(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    int64_t m, int32_t* idx, float* sel_score, int select, void* O, float* w_out,
                                    float* lse_out, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
                                    int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * Decode step with several landmarks per chunk: as hils_decode_step_rq
 * (q_ret may be null) with K_lm_cache [B][H][N_max][m][d] (dt), 1 <= m <= 16;
 * the caller writes the open chunk's m landmark rows before the step.
 */
hils_status hils_decode_step_ml(const void* q, const void* q_ret, const void* k_new, const void* v_new,
                                void* K_cache, void* V_cache, const void* K_lm_cache, int64_t m, int64_t n_ctx,
                                int64_t L_max, void* o, int32_t* idx, float* w, int64_t B, int64_t H, int64_t d,
                                int64_t C, int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * Backward of hils_sparse_attn_fwd_ml (selection held fixed), 1 <= m <= 4:
 * as hils_sparse_attn_bwd_rq with the same K_lm [B][H][N][m][d]; landmark u
 * of a kept chunk takes the share p_u = softmax_u of the chunk's landmark
 * scores of its score gradient, so dK_lm is [B][H][N][m][d] float and dQ (or
 * dQ_ret) gets scale * ds * sum_u p_u K_lm[j][u].
 * Workspace: hils_workspace_size(HILS_OP_BWD, ...).
 */
hils_status hils_sparse_attn_bwd_ml(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    int64_t m, const void* dO, const int32_t* idx, const float* w, const float* lse,
                                    float* dQ, float* dQ_ret, float* dK, float* dV, float* dK_lm, int64_t B,
                                    int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk, float scale,
                                    hils_dtype dt, void* ws, size_t ws_bytes, void* stream);

/*
 * Batched decode over a paged cache (serving shapes: B sequences at their own
 * positions, pages of one chunk).  The same step as hils_decode_step_rq /
 * hils_decode_step_lf (ai-feeds summary "Limitations": the per-step landmark
 * scan; "Method" > "Key modules" items 1-3) for each sequence b at position
 * n_ctx[b], with the caches held in page pools:
 *   K_pages, V_pages : [n_pages][H][64][d] (dt); page p holds, for every head,
 *                      the 64 key / value rows of one chunk
 *   K_lm_pages       : [n_pages][H][m][d] (dt); the m landmark rows of that
 *                      chunk (m = 1: one landmark; m > 1: several landmarks,
 *                      the chunk score is the log-sum-exp of their scores as
 *                      in hils_decode_step_ml)
 *   m                : landmarks per chunk, 1 <= m <= 16 (m > 1 needs
 *                      landmark_free = 0)
 *   page_table       : [B][max_pages] int32 (device): pool page of chunk j of
 *                      sequence b, for every chunk 0 .. n_ctx[b]/64
 *   n_ctx            : [B] int64 (device): each sequence's position; the new
 *                      k_new / v_new row is appended at it
 *   n_ctx_max        : host value >= every n_ctx[b], < max_pages*64; it sizes
 *                      the landmark scan
 *   q, q_ret, k_new, v_new: [B][H][d]; o [B][H][d]; idx, w [B][H][k+1]
 * landmark_free = 1 maintains the open chunk's landmark row as in
 * hils_decode_step_lf.  The table and positions are read on the device:
 * positions, chunk indices and page ids outside their ranges are clamped into
 * them (wrong results, never an access outside the pools); a page must not be
 * shared by two sequences' open chunks.  Workspace:
 * hils_workspace_size(HILS_OP_DECODE, B, H, max_pages*64, d, C, topk).
 */
hils_status hils_decode_step_paged(const void* q, const void* q_ret, const void* k_new, const void* v_new,
                                   void* K_pages, void* V_pages, void* K_lm_pages, int64_t m, const int32_t* page_table,
                                   int64_t n_pages, int64_t max_pages, const int64_t* n_ctx, int64_t n_ctx_max,
                                   int landmark_free, void* o, int32_t* idx, float* w, int64_t B, int64_t H,
                                   int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * Decode step that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and kernels as
 * hils_decode_step without ws / ws_bytes: the step's scratch (per-slice
 * candidate lists and split-K partial outputs, HILS_DECODE_NOALLOC_SCRATCH_BYTES
 * bytes) is a fixed device array of the library, one per GPU, held until the
 * process ends.  Its device address is looked up on the first call on each
 * device (call it once outside graph capture).  B*H is limited to what the
 * array holds (682 at d = 128, 819 at d = 64); larger batches return
 * HILS_ERR_UNSUPPORTED before any HIP call.  Nothing in the array must start
 * at zero; every call rewrites what it reads.  Every call on one GPU shares
 * that GPU's array, which keeps the last call's contents: calls that overlap
 * on one GPU (concurrent streams, or host threads) race and must be
 * serialised by the caller.  Never calls hipMalloc or hipFree.
 */
#define HILS_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
hils_status hils_decode_step_noalloc(const void* q, const void* k_new, const void* v_new, void* K_cache,
                                     void* V_cache, const void* K_lm_cache, int64_t n_ctx, int64_t L_max, void* o,
                                     int32_t* idx, float* w, int64_t B, int64_t H, int64_t d, int64_t C,
                                     int64_t topk, float scale, hils_dtype dt, void* stream);

/*
 * Optional per-kernel timing, for measurement only (off by default; not a
 * step of the method).  While enabled, every kernel an entry point launches
 * carries a start and a stop HIP event that its own dispatch records on the
 * caller's stream (hipExtLaunchKernelGGL), so an interval is the kernel's run;
 * it also includes any time the GPU waited for the host to submit the kernel,
 * so queue the timed launches ahead of the GPU.  Not for use while the stream
 * is being captured into a graph.  hils_profile_enable(on) clears the totals
 * and switches recording on or off.  hils_profile_read waits for the recorded
 * events and returns the number of distinct kernels seen so far; for the first
 * max_kernels of them it writes the kernel name (NUL-terminated, name_stride
 * bytes per entry), the summed duration in milliseconds and the launch count.
 * Any output pointer may be null.  Host-side state only; not thread-safe with
 * concurrent enable/read calls.
 */
void hils_profile_enable(int on);
int hils_profile_read(char* names, int name_stride, double* total_ms, long* calls, int max_kernels);

#ifdef __cplusplus
}
#endif

#endif /* HILS_H */
