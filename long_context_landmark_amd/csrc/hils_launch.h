// Host-side launchers of the HiLS kernels (internal to the library).
// Element type code: 0 = bf16, 1 = fp32.  All launches are asynchronous on
// the given stream and return the launch status.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

// Opt-in per-kernel timing (off unless enabled through the C ABI).  When on, each launch carries a
// start and a stop event that its own dispatch records (hipExtLaunchKernelGGL), so the interval is the
// kernel's execution, without the marker packets of separately recorded events.
namespace prof {
bool make(hipEvent_t* start, hipEvent_t* stop);  // false (and no events) while timing is off
void add(const char* name, hipEvent_t start, hipEvent_t stop);
}  // namespace prof
#define HILS_LAUNCH(name, kernel, grid, block, lds, st, ...)                                      \
  do {                                                                                          \
    hipEvent_t hils_ev_a_ = nullptr, hils_ev_b_ = nullptr;                                      \
    if (::hils::prof::make(&hils_ev_a_, &hils_ev_b_)) {                                         \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, st, hils_ev_a_, hils_ev_b_, 0u, __VA_ARGS__); \
      ::hils::prof::add(name, hils_ev_a_, hils_ev_b_);                                          \
    } else {                                                                                    \
      hipLaunchKernelGGL(kernel, grid, block, lds, st, __VA_ARGS__);                            \
    }                                                                                           \
  } while (0)

hipError_t launch_landmark_scores(int dt, int d, const void* Q, const void* Klm, float* S, int BH, int L, int N,
                                  float scale, hipStream_t st);
// frag_ws: topk_workspace_bytes(BH, N, d) bytes (bf16 only; unused for fp32)
size_t topk_workspace_bytes(int BH, int N, int d);
hipError_t launch_topk(int dt, int d, const void* Q, const void* Klm, void* frag_ws, int32_t* idx, float* sel,
                       float* w, int BH, int L, int N, int k, float scale, hipStream_t st);
// several landmarks per chunk (Klm [BH][N][mlm][d]): the selection kernel forming the log-sum-exp chunk
// scores itself
hipError_t launch_topk_ml(int dt, int d, const void* Q, const void* Klm, int mlm, int32_t* idx, float* sel, float* w,
                          int BH, int L, int N, int k, float scale, hipStream_t st);
// scores and weights of a caller-given selection (slots with idx < 0 are unused)
hipError_t launch_fixed_selection(int dt, int d, const void* Q, const void* Klm, const int32_t* idx, float* sel,
                                  float* w, int BH, int L, int N, int k, float scale, hipStream_t st);

// routing inversion: per (b,h) and chunk j, the list of (query, slot) pairs whose selection holds j
struct RouteBufs {
  int* counts;     // [BH][nseg][N]: per-segment counts, then per-segment offsets
  int* chunk_off;  // [BH][N+1]
  int4* items;     // [BH][max_items]: (chunk, first pair, end pair, -) work items of the chunk-major kernels
  int* n_items;    // [BH]
  int* pairs;      // [BH][L*k]: (t << 5) | slot, grouped by chunk, ascending (t, slot) inside a chunk
  int* pos_of;     // [BH][L][k]: position of pair (t, slot) in pairs, -1 for unused slots (null: not kept)
  int nseg, seg_q, max_items, pairs_per_item;
};
int route_nseg(int L);
int route_seg_q(int L);
int route_max_items(int L, int N, int k, int pairs_per_item);
hipError_t launch_route(const int32_t* idx, const RouteBufs& rb, int BH, int L, int N, int k, hipStream_t st);

// Writes, for every pair at position p of the routing lists, the chunk output (softmax
// attention of the query over the chunk, not yet weighted) partial[bh][p][d] (bf16 for 16-bit
// inputs, fp32 for fp32 inputs) and the chunk log-partition lse_pair[bh][p]: consecutive pairs of a
// work item land in consecutive rows.  trash (d elements) and trash_lse (one float) receive
// the stores of absent pairs.
hipError_t launch_chunk_attn_fwd(int dt, int d, const void* Q, const void* K, const void* V, const RouteBufs& rb,
                                 float* lse_pair, void* partial, void* trash, float* trash_lse,
                                 int BH, int L, int N, int k, float scale, hipStream_t st);
// partial and lse_pair are indexed by pair position (chunk-major, as chunk_attn_fwd writes
// them); pos_of maps (query, slot) to that position
hipError_t launch_own_combine(int dt, int d, const void* Q, const void* K, const void* V, const int* pos_of,
                              const float* w, const void* partial, const float* lse_pair, void* O, float* lse,
                              int BH, int L, int N, int k, float scale, hipStream_t st);
// pairs per chunk-major work item: short sequences favour balance, long ones fewer K/V re-reads
inline int fwd_pairs_per_item(int N) { return N <= 1024 ? 512 : 2048; }

struct DecodeBufs {
  uint64_t* lists;  // [BH][decode_max_slices()][decode_list_len()] best (score, chunk) keys of every slice
  float* part;      // [BH][decode_split()][d] weighted partial outputs of the attention workgroups
};
// cache addressing of a decode step: contiguous (pt == nullptr) or paged (see launch_decode_paged)
struct DecAddr {
  const int32_t* pt;    // page table [B][max_pages]: pool page of each chunk of each sequence
  const int64_t* npos;  // position of each sequence [B]
  int max_pages;
  int H;
  int64_t pages;  // pages in the pool
};
int decode_split();
int decode_slices(int64_t n_ctx);
int decode_max_slices();
int decode_list_len();

struct BwdBufs {
  RouteBufs rb;
  void* dq_part;    // [BH][L][k+1][d] in-chunk dQ contribution of every (query, slot): bf16 for 16-bit
                    // inputs, fp32 for fp32 inputs
  float* Dpart;    // [BH][L][k+1]    D_j = dO_t . o_tj of every (query, slot)
  float* ds;       // [BH][L][k+1]    fusion-score gradient of every (query, slot)
  void* trash;     // d elements: stores of lanes without a pair
  float* trash_f;  // one float, likewise
};
// Qr / dQr: retrieval queries that scored the landmarks and their gradient (both null: Q scored them,
// and dQ takes the whole gradient)
// lf: landmark-free chunks (Klm holds the key means); the score gradients are carried into dK as well,
// and dKlm receives the past chunks' mean gradient
hipError_t launch_bwd(int dt, int d, const void* Q, const void* Qr, const void* K, const void* V, const void* Klm,
                      bool lf, int mlm, const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ,
                      float* dQr, float* dK, float* dV, float* dKlm, int BH, int L, int N, int k, float scale,
                      const BwdBufs& ws, hipStream_t st);
// landmark-free backward tail, per (chunk, head): the mean paths (own slots and the past chunk's dKlm)
// into dK; the own slot's ds against the causal means reaches dQs in dq_reduce
hipError_t launch_lf_bwd(int dt, int d, const void* Qs, const float* ds, const float* dKlm, float* dK, int BH, int L,
                         int N, int k, float scale, hipStream_t st);
// qr: retrieval query for the landmark scores (null: q).  lf: landmark-free chunks, the step writes
// the open chunk's landmark row (the mean of its keys so far) before it is read
// mlm: landmarks per chunk (Klm [BH][Nmax][mlm][d]; the chunk score is the log-sum-exp of theirs)
hipError_t launch_decode(int dt, int d, const void* q, const void* qr, const void* k_new, const void* v_new, void* Kc,
                         void* Vc, const void* Klm, bool lf, int mlm, int64_t n, int64_t Lmax, int64_t Nmax, void* o,
                         int32_t* idx, float* w, int BH, int k, float scale, const DecodeBufs& ws, hipStream_t st);
// decode step of B sequences at their own positions n_ctx[b] (device, <= n_max) over paged caches: page p of
// the pools holds one chunk of 64 rows per head (Kp, Vp: [pages][H][64][d]; Klm_p: [pages][H][mlm][d])
hipError_t launch_decode_paged(int dt, int d, const void* q, const void* qr, const void* k_new, const void* v_new,
                               void* Kp, void* Vp, void* Klm_p, bool lf, int mlm, const int32_t* page_table, int max_pages,
                               int64_t pages, const int64_t* n_ctx, int64_t n_max, int B, int H, void* o,
                               int32_t* idx, float* w, int k, float scale, const DecodeBufs& ws, hipStream_t st);
// several landmarks per chunk (Klm [BH][N][m][d]): the selection (select = 1) or the scores of the caller's
// idx (select = 0), and the weights; the chunk score is the log-sum-exp of its landmark scores
hipError_t launch_ml_selection(int dt, int d, const void* Qs, const void* Klm, int m, int32_t* idx, float* sel,
                               float* w, int BH, int L, int N, int k, int select, float scale, hipStream_t st);
// backward tail of several landmarks per chunk (1 <= m <= 4): dKlm [BH][N][m][d] over each
// chunk's pairs (the slots' score terms of dQs are added by the backward's dq_reduce)
hipError_t launch_ml_bwd(int dt, int d, const void* Qs, const void* Klm, int m, const float* ds, const int* chunk_off,
                         const int* pairs, float* dKlm, int BH, int L, int N, int k, float scale, hipStream_t st);
// landmark-free chunk keys: rows 0..nchunks-1 of Klm ([BH][Nlm][d]) = means of the key rows of each chunk
// (K: [BH][Lk][d])
hipError_t launch_chunk_means(int dt, int d, const void* K, void* Klm, int BH, int64_t Lk, int64_t Nlm, int nchunks,
                              hipStream_t st);
// landmark-free own chunk: after the selection, each query's own-slot score against the mean of its chunk's
// keys up to it, and the fusion weights from the kept past scores (L a multiple of 64)
hipError_t launch_lf_own(int dt, int d, const void* Qs, const void* K, const int32_t* idx, float* sel, float* w,
                         int BH, int L, int k, float scale, hipStream_t st);

}  // namespace hils
