// C ABI of libhils: argument validation, workspace carving and kernel launches.
// Every check runs on the host before any HIP call; see include/hils.h for the
// contract of each entry point.
#include "hils.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "hils_launch.h"

namespace {

thread_local char g_err[512] = "";

hils_status fail(hils_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

hils_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return HILS_OK;
  return fail(HILS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Dims {
  int64_t B, H, L, d, C, k, N;
};

// Shape checks shared by the prefill-shaped entry points.
hils_status check_dims(int64_t B, int64_t H, int64_t L, int64_t d, int64_t C, int64_t k, bool need_k, Dims* out) {
  if (B < 1 || H < 1) return fail(HILS_ERR_INVALID_ARG, "B and H must be >= 1 (got B=%lld H=%lld)", (long long)B, (long long)H);
  if (L < 1) return fail(HILS_ERR_INVALID_ARG, "L must be >= 1 (got %lld)", (long long)L);
  if (C != 64) return fail(HILS_ERR_UNSUPPORTED, "chunk size C must be 64 (got %lld)", (long long)C);
  if (L % C) return fail(HILS_ERR_INVALID_ARG, "L (%lld) must be a multiple of C (%lld)", (long long)L, (long long)C);
  if (d != 64 && d != 128) return fail(HILS_ERR_UNSUPPORTED, "head dim d must be 64 or 128 (got %lld)", (long long)d);
  const int64_t N = L / C;
  if (N > 16384) return fail(HILS_ERR_UNSUPPORTED, "at most 16384 chunks per sequence (got %lld)", (long long)N);
  if (need_k && (k < 1 || k > 16)) return fail(HILS_ERR_UNSUPPORTED, "top-k must be in [1, 16] (got %lld)", (long long)k);
  const int64_t kk = need_k ? k : 0;
  if (B * H * L * (kk + 1) >= (int64_t(1) << 31) || B * H * L * d >= (int64_t(1) << 40))
    return fail(HILS_ERR_UNSUPPORTED, "problem too large for 32-bit pair indexing");
  if (B * H > 65535 * 64) return fail(HILS_ERR_UNSUPPORTED, "B*H too large");
  *out = Dims{B, H, L, d, C, kk, N};
  return HILS_OK;
}

hils_status check_dt(int dt) {
  if (dt != HILS_BF16 && dt != HILS_FP32) return fail(HILS_ERR_INVALID_ARG, "unknown element type %d", dt);
  return HILS_OK;
}

#define REQUIRE_PTR(p)                                                                          \
  do {                                                                                          \
    if (!(p)) return fail(HILS_ERR_INVALID_ARG, "%s must not be null", #p);                     \
    if (!aligned16(p)) return fail(HILS_ERR_INVALID_ARG, "%s must be 16-byte aligned", #p);      \
  } while (0)
#define OPTIONAL_PTR(p)                                                                         \
  do {                                                                                          \
    if ((p) && !aligned16(p)) return fail(HILS_ERR_INVALID_ARG, "%s must be 16-byte aligned", #p); \
  } while (0)

// Workspace carving: a bump allocator over the caller's buffer.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T> T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

struct FwdWs {
  hils::RouteBufs rb;
  void* partial;     // [BH][L*k][d] chunk outputs: bf16, or fp32 for fp32 inputs
  void* trash;       // d elements: stores of absent pairs in the chunk-major kernel
  float* trash_lse;
  float* lse_pair;  // [BH][L*k] chunk log-partition of every pair, in list order
  float* w_tmp;
  void* klm_frag;   // landmarks in fragment order for the selection sweeps
};

size_t carve_route(Carver& cv, const Dims& D, hils::RouteBufs& rb, int ppi) {
  const int64_t BH = D.B * D.H;
  rb.nseg = hils::route_nseg((int)D.L);
  rb.seg_q = hils::route_seg_q((int)D.L);
  rb.pairs_per_item = ppi;
  rb.max_items = hils::route_max_items((int)D.L, (int)D.N, (int)D.k, ppi);
  rb.counts = cv.take<int>((size_t)BH * rb.nseg * D.N);
  rb.chunk_off = cv.take<int>((size_t)BH * (D.N + 1));
  rb.items = cv.take<int4>((size_t)BH * rb.max_items);
  rb.n_items = cv.take<int>((size_t)BH);
  rb.pairs = cv.take<int>((size_t)BH * D.L * D.k);
  rb.pos_of = nullptr;
  return cv.off;
}


// esz: bytes per element of the per-pair intermediate rows (2: 16-bit inputs, 4: fp32 inputs)
size_t carve_fwd(void* base, const Dims& D, FwdWs* ws, int esz) {
  Carver cv(base);
  const int64_t BH = D.B * D.H;
  carve_route(cv, D, ws->rb, hils::fwd_pairs_per_item((int)D.N));
  ws->rb.pos_of = cv.take<int>((size_t)BH * D.L * D.k);
  ws->partial = cv.take<uint8_t>((size_t)BH * D.L * D.k * D.d * esz);
  ws->lse_pair = cv.take<float>((size_t)BH * D.L * D.k);
  ws->w_tmp = cv.take<float>((size_t)BH * D.L * (D.k + 1));
  ws->trash = cv.take<float>((size_t)D.d);
  ws->trash_lse = cv.take<float>(64);
  ws->klm_frag = cv.take<uint8_t>(hils::topk_workspace_bytes((int)BH, (int)D.N, (int)D.d));
  return cv.off;
}

size_t carve_bwd(void* base, const Dims& D, hils::BwdBufs* ws, int esz) {
  Carver cv(base);
  const int64_t BH = D.B * D.H;
  carve_route(cv, D, ws->rb, hils::fwd_pairs_per_item((int)D.N));
  ws->dq_part = cv.take<uint8_t>((size_t)BH * D.L * (D.k + 1) * D.d * esz);
  ws->Dpart = cv.take<float>((size_t)BH * D.L * (D.k + 1));
  ws->ds = cv.take<float>((size_t)BH * D.L * (D.k + 1));
  ws->trash = cv.take<float>((size_t)D.d);
  ws->trash_f = cv.take<float>(64);
  return cv.off;
}

size_t carve_decode(void* base, int64_t BH, int64_t Lmax, int64_t d, int64_t k, hils::DecodeBufs* ws) {
  Carver cv(base);
  ws->lists = cv.take<uint64_t>((size_t)(BH * hils::decode_max_slices() * hils::decode_list_len()));
  ws->part = cv.take<float>((size_t)(BH * hils::decode_split() * d));
  (void)Lmax;
  (void)k;
  return cv.off;
}

hils_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return HILS_OK;
  if (!ws) return fail(HILS_ERR_WORKSPACE, "workspace of %zu bytes required, got null", need);
  if (!aligned16(ws)) return fail(HILS_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (ws_bytes < need) return fail(HILS_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return HILS_OK;
}

}  // namespace

static hils_status fwd_impl(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm, bool lf,
                            int64_t mlm, int32_t* idx, float* sel_score, int select, void* O, float* w_out,
                            float* lse_out, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk,
                            float scale, hils_dtype dt, void* ws, size_t ws_bytes, void* stream);
static hils_status decode_impl(const void* q, const void* q_ret, const void* k_new, const void* v_new, void* K_cache,
                               void* V_cache, const void* K_lm_cache, bool lf, int64_t mlm, int64_t n_ctx, int64_t L_max, void* o,
                               int32_t* idx, float* w, int64_t B, int64_t H, int64_t d, int64_t C, int64_t topk,
                               float scale, hils_dtype dt, void* ws, size_t ws_bytes, void* stream,
                               bool validate_only = false);
static hils_status bwd_impl(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm, bool lf,
                            int64_t mlm, const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ,
                            float* dQ_ret, float* dK, float* dV, float* dK_lm, int64_t B, int64_t H, int64_t L,
                            int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt, void* ws,
                            size_t ws_bytes, void* stream);

extern "C" {

const char* hils_last_error(void) { return g_err; }

int hils_version(void) { return 10000; }

size_t hils_workspace_size(int op, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk) {
  Dims D;
  g_err[0] = 0;
  const int esz = (op & HILS_WS_FP32) ? 4 : 2;
  op &= ~HILS_WS_FP32;
  switch (op) {
    case HILS_OP_SCORES:
      return 0;
    case HILS_OP_TOPK:
      if (check_dims(B, H, L, d, C, topk, true, &D) != HILS_OK) return 0;
      return hils::topk_workspace_bytes((int)(B * H), (int)D.N, (int)d);
    case HILS_OP_FWD: {
      if (check_dims(B, H, L, d, C, topk, true, &D) != HILS_OK) return 0;
      FwdWs ws;
      return carve_fwd(nullptr, D, &ws, esz);
    }
    case HILS_OP_FWD_ML: {  // as the plain forward: no score matrix is formed
      if (check_dims(B, H, L, d, C, topk, true, &D) != HILS_OK) return 0;
      FwdWs ws;
      return carve_fwd(nullptr, D, &ws, esz);
    }
    case HILS_OP_BWD: {
      if (check_dims(B, H, L, d, C, topk, true, &D) != HILS_OK) return 0;
      hils::BwdBufs ws;
      return carve_bwd(nullptr, D, &ws, esz);
    }
    case HILS_OP_DECODE: {
      if (check_dims(B, H, ((L + C - 1) / (C > 0 ? C : 1)) * (C > 0 ? C : 1), d, C, topk, true, &D) != HILS_OK)
        return 0;
      hils::DecodeBufs ws;
      return carve_decode(nullptr, B * H, L, d, topk, &ws);
    }
    default:
      fail(HILS_ERR_INVALID_ARG, "unknown operation code %d", op);
      return 0;
  }
}

hils_status hils_landmark_scores(const void* Q, const void* K_lm, float* S, int64_t B, int64_t H, int64_t L,
                                 int64_t d, int64_t C, float scale, hils_dtype dt, void* stream) {
  Dims D;
  hils_status st;
  if ((st = check_dims(B, H, L, d, C, 0, false, &D)) != HILS_OK) return st;
  if ((st = check_dt(dt)) != HILS_OK) return st;
  REQUIRE_PTR(Q);
  REQUIRE_PTR(K_lm);
  REQUIRE_PTR(S);
  if (!(scale > 0.f)) return fail(HILS_ERR_INVALID_ARG, "scale must be positive");
  if (B * H * L * D.N >= (int64_t(1) << 40)) return fail(HILS_ERR_UNSUPPORTED, "score matrix too large");
  return hip_status(hils::launch_landmark_scores(dt, (int)d, Q, K_lm, S, (int)(B * H), (int)L, (int)D.N, scale,
                                                 (hipStream_t)stream),
                    "hils_landmark_scores");
}

hils_status hils_topk_select(const void* Q, const void* K_lm, int32_t* idx, float* sel_score, float* w, int64_t B,
                             int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt,
                             void* ws, size_t ws_bytes, void* stream) {
  Dims D;
  hils_status st;
  if ((st = check_dims(B, H, L, d, C, topk, true, &D)) != HILS_OK) return st;
  if ((st = check_dt(dt)) != HILS_OK) return st;
  REQUIRE_PTR(Q);
  REQUIRE_PTR(K_lm);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(sel_score);
  OPTIONAL_PTR(w);
  if (!(scale > 0.f)) return fail(HILS_ERR_INVALID_ARG, "scale must be positive");
  if ((st = check_ws(ws, ws_bytes, hils::topk_workspace_bytes((int)(B * H), (int)D.N, (int)d))) != HILS_OK) return st;
  return hip_status(hils::launch_topk(dt, (int)d, Q, K_lm, ws, idx, sel_score, w, (int)(B * H), (int)L, (int)D.N,
                                      (int)topk, scale, (hipStream_t)stream),
                    "hils_topk_select");
}

hils_status hils_sparse_attn_fwd(const void* Q, const void* K, const void* V, const void* K_lm, int32_t* idx,
                                 float* sel_score, int select, void* O, float* w_out, float* lse_out, int64_t B,
                                 int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk, float scale,
                                 hils_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  return hils_sparse_attn_fwd_rq(Q, nullptr, K, V, K_lm, idx, sel_score, select, O, w_out, lse_out, B, H, L, d, C,
                                 topk, scale, dt, ws, ws_bytes, stream);
}

hils_status hils_sparse_attn_fwd_rq(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    int32_t* idx, float* sel_score, int select, void* O, float* w_out,
                                    float* lse_out, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
                                    int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                    void* stream) {
  return fwd_impl(Q, Q_ret, K, V, K_lm, false, 0, idx, sel_score, select, O, w_out, lse_out, B, H, L, d, C, topk,
                  scale, dt, ws, ws_bytes, stream);
}

hils_status hils_sparse_attn_fwd_lf(const void* Q, const void* Q_ret, const void* K, const void* V, void* K_lm_out,
                                    int32_t* idx, float* sel_score, int select, void* O, float* w_out,
                                    float* lse_out, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
                                    int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                    void* stream) {
  return fwd_impl(Q, Q_ret, K, V, K_lm_out, true, 0, idx, sel_score, select, O, w_out, lse_out, B, H, L, d, C, topk,
                  scale, dt, ws, ws_bytes, stream);
}

hils_status hils_sparse_attn_fwd_ml(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    int64_t m, int32_t* idx, float* sel_score, int select, void* O, float* w_out,
                                    float* lse_out, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
                                    int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (m < 1 || m > 16) return fail(HILS_ERR_UNSUPPORTED, "landmarks per chunk must be in [1, 16] (got %lld)",
                                   (long long)m);
  return fwd_impl(Q, Q_ret, K, V, K_lm, false, m, idx, sel_score, select, O, w_out, lse_out, B, H, L, d, C, topk,
                  scale, dt, ws, ws_bytes, stream);
}

hils_status hils_chunk_means(const void* K, void* K_lm, int64_t B, int64_t H, int64_t L_k, int64_t N_lm,
                             int64_t n_chunks, int64_t d, int64_t C, hils_dtype dt, void* stream) {
  hils_status st;
  if (C != 64) return fail(HILS_ERR_UNSUPPORTED, "chunk size C must be 64 (got %lld)", (long long)C);
  if (d != 64 && d != 128) return fail(HILS_ERR_UNSUPPORTED, "head dim must be 64 or 128 (got %lld)", (long long)d);
  if ((st = check_dt(dt)) != HILS_OK) return st;
  if (B < 1 || H < 1 || B * H > 65535) return fail(HILS_ERR_INVALID_ARG, "B and H must be >= 1 with B*H <= 65535");
  if (n_chunks < 0 || n_chunks * C > L_k || n_chunks > N_lm || n_chunks > 65535)
    return fail(HILS_ERR_INVALID_ARG, "n_chunks (%lld) must be in [0, min(L_k/C, N_lm, 65535)]", (long long)n_chunks);
  REQUIRE_PTR(K);
  REQUIRE_PTR(K_lm);
  return hip_status(hils::launch_chunk_means(dt, (int)d, K, K_lm, (int)(B * H), L_k, N_lm, (int)n_chunks,
                                             (hipStream_t)stream),
                    "hils_chunk_means");
}

}  // extern "C"

static hils_status fwd_impl(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm, bool lf,
                            int64_t mlm, int32_t* idx, float* sel_score, int select, void* O, float* w_out,
                            float* lse_out, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk,
                            float scale, hils_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  Dims D;
  hils_status st;
  if ((st = check_dims(B, H, L, d, C, topk, true, &D)) != HILS_OK) return st;
  if ((st = check_dt(dt)) != HILS_OK) return st;
  REQUIRE_PTR(Q);
  OPTIONAL_PTR(Q_ret);
  REQUIRE_PTR(K);
  REQUIRE_PTR(V);
  REQUIRE_PTR(K_lm);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(sel_score);
  REQUIRE_PTR(O);
  OPTIONAL_PTR(w_out);
  OPTIONAL_PTR(lse_out);
  if (select != 0 && select != 1) return fail(HILS_ERR_INVALID_ARG, "select must be 0 or 1");
  if (!(scale > 0.f)) return fail(HILS_ERR_INVALID_ARG, "scale must be positive");
  FwdWs W;
  const int esz = dt == HILS_FP32 ? 4 : 2;
  const size_t need = carve_fwd(nullptr, D, &W, esz);
  if ((st = check_ws(ws, ws_bytes, need)) != HILS_OK) return st;
  carve_fwd(ws, D, &W, esz);
  const int BH = (int)(B * H), iL = (int)L, iN = (int)D.N, ik = (int)topk, id = (int)d;
  hipStream_t s = (hipStream_t)stream;
  float* w = w_out ? w_out : W.w_tmp;
  hipError_t e;
  // the landmark scores (selection and fusion weights) use the retrieval queries when given
  const void* Qs = Q_ret ? Q_ret : Q;
  // landmark-free chunks: the landmarks are the chunks' key means, formed here
  if (lf && (e = hils::launch_chunk_means(dt, id, K, (void*)K_lm, BH, L, D.N, iN, s)) != hipSuccess)
    return hip_status(e, "hils_sparse_attn_fwd: chunk means");
  if (mlm > 0)
    e = hils::launch_ml_selection(dt, id, Qs, K_lm, (int)mlm, idx, sel_score, w, BH, iL, iN, ik, select, scale, s);
  else if (select) e = hils::launch_topk(dt, id, Qs, K_lm, W.klm_frag, idx, sel_score, w, BH, iL, iN, ik, scale, s);
  else e = hils::launch_fixed_selection(dt, id, Qs, K_lm, idx, sel_score, w, BH, iL, iN, ik, scale, s);
  if (e != hipSuccess) return hip_status(e, "hils_sparse_attn_fwd: selection");
  // ... and the own chunk is scored by the mean of its keys up to the query
  if (lf && (e = hils::launch_lf_own(dt, id, Qs, K, idx, sel_score, w, BH, iL, ik, scale, s)) != hipSuccess)
    return hip_status(e, "hils_sparse_attn_fwd: own chunk landmarks");
  if ((e = hils::launch_route(idx, W.rb, BH, iL, iN, ik, s)) != hipSuccess)
    return hip_status(e, "hils_sparse_attn_fwd: routing");
  if ((e = hils::launch_chunk_attn_fwd(dt, id, Q, K, V, W.rb, W.lse_pair, W.partial, W.trash, W.trash_lse, BH, iL,
                                       iN, ik, scale, s)) != hipSuccess)
    return hip_status(e, "hils_sparse_attn_fwd: chunk attention");
  if ((e = hils::launch_own_combine(dt, id, Q, K, V, W.rb.pos_of, w, W.partial, W.lse_pair, O, lse_out, BH, iL, iN,
                                    ik, scale, s)) != hipSuccess)
    return hip_status(e, "hils_sparse_attn_fwd: own chunk and fusion");
  return HILS_OK;
}

extern "C" {

hils_status hils_decode_step(const void* q, const void* k_new, const void* v_new, void* K_cache, void* V_cache,
                             const void* K_lm_cache, int64_t n_ctx, int64_t L_max, void* o, int32_t* idx, float* w,
                             int64_t B, int64_t H, int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt,
                             void* ws, size_t ws_bytes, void* stream) {
  return hils_decode_step_rq(q, nullptr, k_new, v_new, K_cache, V_cache, K_lm_cache, n_ctx, L_max, o, idx, w, B, H,
                             d, C, topk, scale, dt, ws, ws_bytes, stream);
}

hils_status hils_decode_step_rq(const void* q, const void* q_ret, const void* k_new, const void* v_new,
                                void* K_cache, void* V_cache, const void* K_lm_cache, int64_t n_ctx, int64_t L_max,
                                void* o, int32_t* idx, float* w, int64_t B, int64_t H, int64_t d, int64_t C,
                                int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                void* stream) {
  return decode_impl(q, q_ret, k_new, v_new, K_cache, V_cache, K_lm_cache, false, 1, n_ctx, L_max, o, idx, w, B, H, d,
                     C, topk, scale, dt, ws, ws_bytes, stream);
}

hils_status hils_decode_step_lf(const void* q, const void* q_ret, const void* k_new, const void* v_new,
                                void* K_cache, void* V_cache, void* K_lm_cache, int64_t n_ctx, int64_t L_max,
                                void* o, int32_t* idx, float* w, int64_t B, int64_t H, int64_t d, int64_t C,
                                int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                void* stream) {
  return decode_impl(q, q_ret, k_new, v_new, K_cache, V_cache, K_lm_cache, true, 1, n_ctx, L_max, o, idx, w, B, H, d,
                     C, topk, scale, dt, ws, ws_bytes, stream);
}

hils_status hils_decode_step_ml(const void* q, const void* q_ret, const void* k_new, const void* v_new,
                                void* K_cache, void* V_cache, const void* K_lm_cache, int64_t m, int64_t n_ctx,
                                int64_t L_max, void* o, int32_t* idx, float* w, int64_t B, int64_t H, int64_t d,
                                int64_t C, int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                void* stream) {
  if (m < 1 || m > 16) return fail(HILS_ERR_UNSUPPORTED, "landmarks per chunk must be in [1, 16] (got %lld)",
                                   (long long)m);
  return decode_impl(q, q_ret, k_new, v_new, K_cache, V_cache, K_lm_cache, false, m, n_ctx, L_max, o, idx, w, B, H,
                     d, C, topk, scale, dt, ws, ws_bytes, stream);
}

}  // extern "C"

static hils_status decode_impl(const void* q, const void* q_ret, const void* k_new, const void* v_new, void* K_cache,
                               void* V_cache, const void* K_lm_cache, bool lf, int64_t mlm, int64_t n_ctx, int64_t L_max, void* o,
                               int32_t* idx, float* w, int64_t B, int64_t H, int64_t d, int64_t C, int64_t topk,
                               float scale, hils_dtype dt, void* ws, size_t ws_bytes, void* stream,
                               bool validate_only) {
  Dims D;
  hils_status st;
  if (L_max < 1) return fail(HILS_ERR_INVALID_ARG, "L_max must be >= 1 (got %lld)", (long long)L_max);
  if (C != 64) return fail(HILS_ERR_UNSUPPORTED, "chunk size C must be 64 (got %lld)", (long long)C);
  const int64_t Nmax = (L_max + C - 1) / C;
  if ((st = check_dims(B, H, Nmax * C, d, C, topk, true, &D)) != HILS_OK) return st;
  if ((st = check_dt(dt)) != HILS_OK) return st;
  if (n_ctx < 0 || n_ctx >= L_max)
    return fail(HILS_ERR_INVALID_ARG, "n_ctx (%lld) must be in [0, L_max=%lld)", (long long)n_ctx, (long long)L_max);
  REQUIRE_PTR(q);
  OPTIONAL_PTR(q_ret);
  REQUIRE_PTR(k_new);
  REQUIRE_PTR(v_new);
  REQUIRE_PTR(K_cache);
  REQUIRE_PTR(V_cache);
  REQUIRE_PTR(K_lm_cache);
  REQUIRE_PTR(o);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(w);
  if (!(scale > 0.f)) return fail(HILS_ERR_INVALID_ARG, "scale must be positive");
  if (validate_only) return HILS_OK;
  hils::DecodeBufs W;
  const size_t need = carve_decode(nullptr, B * H, L_max, d, topk, &W);
  if ((st = check_ws(ws, ws_bytes, need)) != HILS_OK) return st;
  carve_decode(ws, B * H, L_max, d, topk, &W);
  return hip_status(hils::launch_decode(dt, (int)d, q, q_ret, k_new, v_new, K_cache, V_cache, K_lm_cache, lf, (int)mlm,
                                        n_ctx,
                                        L_max, Nmax, o, idx, w, (int)(B * H), (int)topk, scale, W,
                                        (hipStream_t)stream),
                    "hils_decode_step");
}

extern "C" {

hils_status hils_sparse_attn_bwd(const void* Q, const void* K, const void* V, const void* K_lm, const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ,
                                 float* dK, float* dV, float* dK_lm, int64_t B, int64_t H, int64_t L, int64_t d,
                                 int64_t C, int64_t topk, float scale, hils_dtype dt, void* ws, size_t ws_bytes,
                                 void* stream) {
  return hils_sparse_attn_bwd_rq(Q, nullptr, K, V, K_lm, dO, idx, w, lse, dQ, nullptr, dK, dV, dK_lm, B, H, L, d, C,
                                 topk, scale, dt, ws, ws_bytes, stream);
}

hils_status hils_sparse_attn_bwd_rq(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ,
                                    float* dQ_ret, float* dK, float* dV, float* dK_lm, int64_t B, int64_t H,
                                    int64_t L, int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt,
                                    void* ws, size_t ws_bytes, void* stream) {
  return bwd_impl(Q, Q_ret, K, V, K_lm, false, 0, dO, idx, w, lse, dQ, dQ_ret, dK, dV, dK_lm, B, H, L, d, C, topk, scale,
                  dt, ws, ws_bytes, stream);
}

hils_status hils_sparse_attn_bwd_lf(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ,
                                    float* dQ_ret, float* dK, float* dV, float* dK_lm, int64_t B, int64_t H,
                                    int64_t L, int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt,
                                    void* ws, size_t ws_bytes, void* stream) {
  return bwd_impl(Q, Q_ret, K, V, K_lm, true, 0, dO, idx, w, lse, dQ, dQ_ret, dK, dV, dK_lm, B, H, L, d, C, topk,
                  scale, dt, ws, ws_bytes, stream);
}

hils_status hils_sparse_attn_bwd_ml(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm,
                                    int64_t m, const void* dO, const int32_t* idx, const float* w, const float* lse,
                                    float* dQ, float* dQ_ret, float* dK, float* dV, float* dK_lm, int64_t B,
                                    int64_t H, int64_t L, int64_t d, int64_t C, int64_t topk, float scale,
                                    hils_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  if (m < 1 || m > 4)
    return fail(HILS_ERR_UNSUPPORTED, "backward: landmarks per chunk must be in [1, 4] (got %lld)", (long long)m);
  return bwd_impl(Q, Q_ret, K, V, K_lm, false, m, dO, idx, w, lse, dQ, dQ_ret, dK, dV, dK_lm, B, H, L, d, C, topk,
                  scale, dt, ws, ws_bytes, stream);
}

}  // extern "C"

static hils_status bwd_impl(const void* Q, const void* Q_ret, const void* K, const void* V, const void* K_lm, bool lf,
                            int64_t mlm, const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ,
                            float* dQ_ret, float* dK, float* dV, float* dK_lm, int64_t B, int64_t H, int64_t L,
                            int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt, void* ws,
                            size_t ws_bytes, void* stream) {
  Dims D;
  hils_status st;
  if ((st = check_dims(B, H, L, d, C, topk, true, &D)) != HILS_OK) return st;
  if ((st = check_dt(dt)) != HILS_OK) return st;
  if ((Q_ret == nullptr) != (dQ_ret == nullptr))
    return fail(HILS_ERR_INVALID_ARG, "Q_ret and dQ_ret must be given together");
  OPTIONAL_PTR(Q_ret);
  OPTIONAL_PTR(dQ_ret);
  REQUIRE_PTR(Q);
  REQUIRE_PTR(K);
  REQUIRE_PTR(V);
  REQUIRE_PTR(K_lm);
  REQUIRE_PTR(dO);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(w);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(dQ);
  REQUIRE_PTR(dK);
  REQUIRE_PTR(dV);
  REQUIRE_PTR(dK_lm);
  if (!(scale > 0.f)) return fail(HILS_ERR_INVALID_ARG, "scale must be positive");
  hils::BwdBufs W;
  const int esz = dt == HILS_FP32 ? 4 : 2;
  const size_t need = carve_bwd(nullptr, D, &W, esz);
  if ((st = check_ws(ws, ws_bytes, need)) != HILS_OK) return st;
  carve_bwd(ws, D, &W, esz);
  return hip_status(hils::launch_bwd(dt, (int)d, Q, Q_ret, K, V, K_lm, lf, (int)mlm, dO, idx, w, lse, dQ, dQ_ret, dK, dV, dK_lm,
                                     (int)(B * H), (int)L, (int)D.N, (int)topk, scale, W, (hipStream_t)stream),
                    "hils_sparse_attn_bwd");
}

extern "C" {

hils_status hils_decode_step_paged(const void* q, const void* q_ret, const void* k_new, const void* v_new,
                                   void* K_pages, void* V_pages, void* K_lm_pages, int64_t m, const int32_t* page_table,
                                   int64_t n_pages, int64_t max_pages, const int64_t* n_ctx, int64_t n_ctx_max,
                                   int landmark_free, void* o, int32_t* idx, float* w, int64_t B, int64_t H,
                                   int64_t d, int64_t C, int64_t topk, float scale, hils_dtype dt, void* ws,
                                   size_t ws_bytes, void* stream) {
  Dims D;
  hils_status st;
  if (C != 64) return fail(HILS_ERR_UNSUPPORTED, "chunk size C must be 64 (got %lld)", (long long)C);
  if (max_pages < 1) return fail(HILS_ERR_INVALID_ARG, "max_pages must be >= 1 (got %lld)", (long long)max_pages);
  if (n_pages < 1) return fail(HILS_ERR_INVALID_ARG, "n_pages must be >= 1 (got %lld)", (long long)n_pages);
  const int64_t L_max = max_pages * C;
  if ((st = check_dims(B, H, L_max, d, C, topk, true, &D)) != HILS_OK) return st;
  if ((st = check_dt(dt)) != HILS_OK) return st;
  if (n_ctx_max < 0 || n_ctx_max >= L_max)
    return fail(HILS_ERR_INVALID_ARG, "n_ctx_max (%lld) must be in [0, max_pages*C=%lld)", (long long)n_ctx_max,
                (long long)L_max);
  if (landmark_free != 0 && landmark_free != 1) return fail(HILS_ERR_INVALID_ARG, "landmark_free must be 0 or 1");
  if (m < 1 || m > 16) return fail(HILS_ERR_UNSUPPORTED, "landmarks per chunk must be in [1, 16] (got %lld)",
                                   (long long)m);
  if (m > 1 && landmark_free) return fail(HILS_ERR_INVALID_ARG, "landmark-free chunks take one landmark per chunk");
  REQUIRE_PTR(q);
  OPTIONAL_PTR(q_ret);
  REQUIRE_PTR(k_new);
  REQUIRE_PTR(v_new);
  REQUIRE_PTR(K_pages);
  REQUIRE_PTR(V_pages);
  REQUIRE_PTR(K_lm_pages);
  REQUIRE_PTR(page_table);
  REQUIRE_PTR(n_ctx);
  REQUIRE_PTR(o);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(w);
  if (!(scale > 0.f)) return fail(HILS_ERR_INVALID_ARG, "scale must be positive");
  hils::DecodeBufs W;
  const size_t need = carve_decode(nullptr, B * H, L_max, d, topk, &W);
  if ((st = check_ws(ws, ws_bytes, need)) != HILS_OK) return st;
  carve_decode(ws, B * H, L_max, d, topk, &W);
  return hip_status(hils::launch_decode_paged(dt, (int)d, q, q_ret, k_new, v_new, K_pages, V_pages, K_lm_pages,
                                              landmark_free != 0, (int)m, page_table, (int)max_pages, n_pages, n_ctx,
                                              n_ctx_max, (int)B, (int)H, o, idx, w, (int)topk, scale, W,
                                              (hipStream_t)stream),
                    "hils_decode_step_paged");
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Decode step without a caller workspace: the step's scratch (the per-slice candidate lists and
// the split-K partial outputs) lives in a file-scope device array of fixed size, one copy per GPU,
// held until the process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is looked up once per device (with that device current) and only
// that address is ever handed to kernels.
namespace {
constexpr size_t NOALLOC_SCRATCH_BYTES = HILS_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[NOALLOC_MAX_DEVICES] = {};
}  // namespace

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

// Device address of this device's scratch array (looked up on the first call on the device).
static hils_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hils_decode_step_noalloc: hipGetDevice");
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return fail(HILS_ERR_UNSUPPORTED, "hils_decode_step_noalloc: device ordinal %d above %d", dev,
                NOALLOC_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hils_decode_step_noalloc: hipGetSymbolAddress");
    if (!ptr || ((uintptr_t)ptr & 255u))
      return fail(HILS_ERR_HIP, "hils_decode_step_noalloc: scratch array has no usable device address");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return HILS_OK;
}

extern "C" {

hils_status hils_decode_step_noalloc(const void* q, const void* k_new, const void* v_new, void* K_cache,
                                     void* V_cache, const void* K_lm_cache, int64_t n_ctx, int64_t L_max, void* o,
                                     int32_t* idx, float* w, int64_t B, int64_t H, int64_t d, int64_t C,
                                     int64_t topk, float scale, hils_dtype dt, void* stream) {
  // the workspace the plain step would need must fit the scratch array; checked before any HIP call
  if (B >= 1 && H >= 1 && B * H <= (int64_t(1) << 30) && (d == 64 || d == 128)) {
    hils::DecodeBufs W;
    const size_t need = carve_decode(nullptr, B * H, L_max, d, topk, &W);
    if (need > NOALLOC_SCRATCH_BYTES)
      return fail(HILS_ERR_UNSUPPORTED,
                  "hils_decode_step_noalloc: B*H = %lld needs %zu bytes of scratch, above the fixed %zu bytes; "
                  "use hils_decode_step with a workspace",
                  (long long)(B * H), need, NOALLOC_SCRATCH_BYTES);
  }
  // argument checks of the plain step (null workspace pointers: it would reject a real workspace need)
  hils_status st = decode_impl(q, nullptr, k_new, v_new, K_cache, V_cache, K_lm_cache, false, 1, n_ctx, L_max, o,
                               idx, w, B, H, d, C, topk, scale, dt, nullptr, 0, nullptr, /*validate_only=*/true);
  if (st != HILS_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != HILS_OK) return st;
  return decode_impl(q, nullptr, k_new, v_new, K_cache, V_cache, K_lm_cache, false, 1, n_ctx, L_max, o, idx, w, B, H,
                     d, C, topk, scale, dt, ws, NOALLOC_SCRATCH_BYTES, stream, false);
}

}  // extern "C"
