// One decode step of HiLS attention: append, landmark scan, top-k, split-K
// chunk attention and fusion for a single new query per (b,h).
//
// Passages: "Hierarchical Sparse Attention Done Right" (ai-feeds summary),
// "Limitations" (at every decode step each chunk's landmark is scored, a cost
// linear in the context) and "Method" > "Key modules" items 1-3; the
// paper.oopus.info review, sections 3-4 (single-GPU bf16 decode at long
// context).  The operator is the prefill one for the query at position n:
// candidates are the completed chunks j < n/64, the open chunk n/64 is its own
// chunk (keys 64*(n/64) .. n).
//
// The step is bound by HBM reads of the landmark rows (every step reads all of
// them).  decode_scan streams them with 16-byte coalesced loads over many
// workgroups; each workgroup scores 256 chunks and writes only its 16 best
// (score, chunk) keys, sorted.  The top-m of the context is the top-m of the
// union of these lists, since m <= 16.  decode_attend runs DEC_SPLIT = 8
// workgroups of two wavefronts per head: wave 0 of every workgroup merges the
// lists (the m-th largest of a few list heads bounds the answer from below; the
// keys above the bound are compacted with ballots and sorted exactly) and forms
// the fusion weights, while the second wave of workgroup 0 already attends to
// the open chunk, which needs no selection.  The kept chunks are then split over
// the 16 wavefronts of the eight workgroups (split-K), each reading its chunk's
// keys and values with 16-byte loads; every workgroup writes its weighted
// partial sum, and decode_fuse adds the eight partials of a head in order.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

constexpr int DEC_ROWS = 256;                          // landmark rows per scan workgroup
constexpr int DEC_LIST = 16;                           // keys kept per slice: the largest k accepted
constexpr int DEC_MAX_SLICES = 16384 / DEC_ROWS;       // slices at the library's chunk limit

int decode_slices(int64_t n_ctx) { return (int)((n_ctx / 64 + DEC_ROWS - 1) / DEC_ROWS); }

// Row addressing of the caches (PG = paged).  Contiguous caches: the rows of (b,h) start at
// bh*Lmax, its landmarks at bh*Nmax, one position n for every sequence.  Paged caches (serving
// caches whose pages are chunks): chunk j of sequence b lives in pool page pt[b][j], whose rows
// for head h start at (page*H + h)*64 and whose landmark row is page*H + h; each sequence has its
// own position npos[b].  Positions, chunk indices and page ids are clamped into the table and the
// pool, so a bad table gives wrong results but no access outside the arrays.
template <bool PG>
__device__ __forceinline__ int64_t dec_pos(const DecAddr& a, int bh, int64_t n) {
  if (!PG) return n;
  const int64_t v = a.npos[bh / a.H];
  return v < 0 ? 0 : (v > (int64_t)a.max_pages * 64 - 1 ? (int64_t)a.max_pages * 64 - 1 : v);
}
__device__ __forceinline__ int64_t dec_page_row(const DecAddr& a, int bh, int j) {
  const int b = bh / a.H, h = bh - b * a.H;
  j = j < 0 ? 0 : (j >= a.max_pages ? a.max_pages - 1 : j);
  int64_t p = a.pt[(int64_t)b * a.max_pages + j];
  p = p < 0 ? 0 : (p >= a.pages ? a.pages - 1 : p);
  return p * a.H + h;
}
// first K/V row of chunk j of (b,h), and its landmark row
template <bool PG>
__device__ __forceinline__ int64_t dec_chunk_row(const DecAddr& a, int bh, int j, int64_t Lmax) {
  return PG ? dec_page_row(a, bh, j) * 64 : (int64_t)bh * Lmax + (int64_t)j * 64;
}
template <bool PG>
__device__ __forceinline__ int64_t dec_lm_row(const DecAddr& a, int bh, int j, int64_t Nmax) {
  return PG ? dec_page_row(a, bh, j) : (int64_t)bh * Nmax + j;
}
int decode_max_slices() { return DEC_MAX_SLICES; }
int decode_list_len() { return DEC_LIST; }

// Lanes 0 .. n-1 hold keys (n <= 64, wave-uniform), the others 0: sorts them descending over
// the fewest lanes that hold them (a 16- or 32-lane network has 10 or 15 stages, not 21).
__device__ __forceinline__ uint64_t sort_first_desc(uint64_t v, int n, int lane) {
  if (n <= 16) return wave_sort_desc<uint64_t, 16>(v, lane);
  if (n <= 32) return wave_sort_desc<uint64_t, 32>(v, lane);
  return wave_sort_desc<uint64_t, 64>(v, lane);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Exclusive prefix sum over the lanes of counts in [0, 32), and their total, from five ballots.
__device__ __forceinline__ int wave_excl_prefix_small(int v, int& total) {
  int pre = 0;
  total = 0;
#pragma unroll
  for (int b = 0; b < 5; ++b) {
    const uint64_t bits = __ballot((v >> b) & 1);
    pre += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u)) << b;
    total += __popcll(bits) << b;
  }
  return pre;
}

// LF (landmark-free chunks): the appending workgroup also writes the open chunk's landmark row,
// the mean of its keys so far (rows c*64 .. n-1 from the cache, row n from k_new), rounded to the
// element type; the scan reads only rows of earlier chunks, decode_attend reads this one.  With LF
// the grid has one workgroup more than there are slices, and that last one appends (so the slices
// do not wait for the mean).
template <typename T, int D, bool LF, bool PG, bool ML>
__global__ __launch_bounds__(256) void decode_scan_kernel(const T* __restrict__ q, const T* __restrict__ k_new,
                                                          const T* __restrict__ v_new, T* __restrict__ Kc,
                                                          T* __restrict__ Vc, const T* __restrict__ Klm,
                                                          T* __restrict__ Klm_w, uint64_t* __restrict__ lists,
                                                          int64_t n_in, int64_t Lmax, int64_t Nmax, float scale,
                                                          DecAddr A, int mlm) {
  constexpr int EPP = 16 / Elem<T>::bytes;  // elements per 16-byte piece
  constexpr int PIECES = D / EPP;           // pieces per row
  constexpr int RPR = 256 / PIECES;         // rows per round
  constexpr int ROUNDS = DEC_ROWS / RPR;
  const int s = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int64_t n = dec_pos<PG>(A, bh, n_in);
  const int c = (int)(n / 64);
  if (LF ? s == (int)gridDim.x - 1 : s == 0) {
    // append the new key and value (idempotent)
    const int64_t r0 = dec_chunk_row<PG>(A, bh, c, Lmax);
    const int64_t rn = r0 + (n - (int64_t)c * 64);
    for (int e = tid; e < D; e += 256) {
      Kc[rn * D + e] = k_new[(int64_t)bh * D + e];
      Vc[rn * D + e] = v_new[(int64_t)bh * D + e];
    }
    if (LF) {
      constexpr int G = 256 / D;
      __shared__ float lfp[G][D];
      const int e = tid % D, g = tid / D;
      const int cnt = (int)(n - (int64_t)c * 64);  // cached rows of the open chunk before row n
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 64 / G; ++i) {
        const int r = g + i * G;
        if (r < cnt) acc += Elem<T>::to_f32(Kc, (r0 + r) * D + e);
      }
      lfp[g][e] = acc;
      __syncthreads();
      if (g == 0) {
        float sum = Elem<T>::to_f32(k_new, (int64_t)bh * D + e);
#pragma unroll
        for (int i = 0; i < G; ++i) sum += lfp[i][e];
        Elem<T>::store(Klm_w, dec_lm_row<PG>(A, bh, c, Nmax) * D + e, sum / (float)(cnt + 1));
      }
    }
  }
  const int j0 = s * DEC_ROWS;
  if (j0 >= c) return;
  const int piece = tid % PIECES, rr = tid / PIECES;
  float qv[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) qv[e] = Elem<T>::to_f32(q, (int64_t)bh * D + piece * EPP + e);
  // ML: mlm landmarks per chunk (rows lm*mlm + u), the chunk score is the log-sum-exp of their scores;
  // otherwise one landmark row per chunk
  const int nlm = ML ? mlm : 1;
  float mx[ROUNDS], zz[ROUNDS];
  for (int u = 0; u < nlm; ++u) {
    int4 raw[ROUNDS];
#pragma unroll
    for (int round = 0; round < ROUNDS; ++round) {
      const int j = j0 + round * RPR + rr;
      const int64_t lr = PG ? dec_lm_row<PG>(A, bh, j, Nmax) : (int64_t)bh * Nmax + j;
      const T* rp = Klm + (lr * nlm + u) * D + piece * EPP;
      raw[round] = j < c ? *reinterpret_cast<const int4*>(rp) : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int round = 0; round < ROUNDS; ++round) {
      T vals[EPP];
      __builtin_memcpy(vals, &raw[round], 16);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPP; ++e) dot += qv[e] * Elem<T>::to_f32(vals, e);
#pragma unroll
      for (int m = 1; m < PIECES; m <<= 1) dot += lane_xor(dot, m);
      const float a = scale * dot;
      if (u == 0) {
        mx[round] = a;
        zz[round] = 1.f;
      } else if (a > mx[round]) {
        zz[round] = zz[round] * __expf(mx[round] - a) + 1.f;
        mx[round] = a;
      } else {
        zz[round] += __expf(a - mx[round]);
      }
    }
  }
  __shared__ __align__(16) float sc[DEC_ROWS];
#pragma unroll
  for (int round = 0; round < ROUNDS; ++round)
    if (piece == 0) sc[round * RPR + rr] = ML ? mx[round] + __logf(zz[round]) : mx[round];
  __syncthreads();
  if (tid >= 64) return;
  // The slice's DEC_LIST best keys, by one wave.  Lane l holds scores 4l..4l+3.  The
  // DEC_LIST-th largest of the 64 group maxima bounds the DEC_LIST-th largest score from
  // below (those groups hold that many distinct scores at or above it), so only scores
  // at or above it are sorted as keys.  Order bits of the scores (0 = no chunk) are
  // compared as integers, which is the order of the keys' upper halves.
  const int lane = tid;
  const int nval = min(DEC_ROWS, c - j0);
  const float4 v4 = reinterpret_cast<const float4*>(sc)[lane];
  const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
  uint32_t ob[4];
  uint32_t gmx = 0u;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ob[u] = 4 * lane + u < nval ? ordered_bits(vv[u] + 0.0f) : 0u;
    gmx = max(gmx, ob[u]);
  }
  const uint32_t tau = (uint32_t)__builtin_amdgcn_readlane((int)wave_sort_desc<uint32_t>(gmx, lane), DEC_LIST - 1);
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) cnt += (ob[u] != 0u && ob[u] >= tau) ? 1 : 0;
  int total;
  const int pre = wave_excl_prefix_small(cnt, total);
  __shared__ uint64_t surv[64];
  uint64_t* out = lists + ((int64_t)bh * DEC_MAX_SLICES + s) * DEC_LIST;
  if (total <= 64) {
    int p = pre;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (ob[u] != 0u && ob[u] >= tau) surv[p++] = make_key(vv[u], j0 + 4 * lane + u);
    __builtin_amdgcn_wave_barrier();
    const uint64_t key = sort_first_desc(lane < total ? surv[lane] : 0ull, total, lane);
    if (lane < DEC_LIST) out[lane] = key;
  } else {
    // many scores tied at the bound: a tournament between the lanes' sorted quadruples
    uint64_t kq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kq[u] = ob[u] != 0u ? make_key(vv[u], j0 + 4 * lane + u) : 0ull;
    cmpswap_desc(kq[0], kq[1]);
    cmpswap_desc(kq[2], kq[3]);
    cmpswap_desc(kq[0], kq[2]);
    cmpswap_desc(kq[1], kq[3]);
    cmpswap_desc(kq[1], kq[2]);
    int ptr = 0;
    for (int r = 0; r < DEC_LIST; ++r) {
      const uint64_t head = ptr == 0 ? kq[0] : ptr == 1 ? kq[1] : ptr == 2 ? kq[2] : ptr == 3 ? kq[3] : 0ull;
      uint64_t best = head;
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) {
        const uint64_t o = shfl_xor_u64(best, msk);
        best = o > best ? o : best;
      }
      if (lane == 0) out[r] = best;
      if (head == best && best != 0ull) ++ptr;
    }
  }
}

// top[0..m-1] = the m best keys of the union of S sorted lists of DEC_LIST keys
// (0 = no chunk).  Run by one full wave; lane l holds list l.  The m-th largest
// of the first R = ceil(m/S) keys of every list bounds the m-th best key from below
// (S*R >= m distinct keys), so only keys at or above it take part in the exact sort;
// the bound is taken on the keys' upper halves (the score order bits), which can only
// let in more keys.  When more than 64 keys reach it, m rounds of a tournament between
// the list heads give the same answer.
// The lane's list (lane < S) and its bound key's upper half, requested ahead of other work.
struct MergeIn {
  uint32_t bhi;
  uint64_t mine[DEC_LIST];
};
__device__ __forceinline__ void merge_load(const uint64_t* __restrict__ lists, int S, int m, int lane, MergeIn& in) {
  const int R = (m + S - 1) / S;
  const int nb = S * R;  // <= 64: S if S >= m, else below m + S
  const uint32_t* hi_words = reinterpret_cast<const uint32_t*>(lists);
  in.bhi = lane < nb ? hi_words[2 * ((lane % S) * DEC_LIST + lane / S) + 1] : 0u;
  const ulonglong2* lp = reinterpret_cast<const ulonglong2*>(lists + lane * DEC_LIST);
#pragma unroll
  for (int u = 0; u < DEC_LIST / 2; ++u) {
    const ulonglong2 v2 = lane < S ? lp[u] : make_ulonglong2(0ull, 0ull);
    in.mine[2 * u] = v2.x;
    in.mine[2 * u + 1] = v2.y;
  }
}
__device__ void wave_merge_lists(const MergeIn& in, int m, uint64_t* top, uint64_t* surv, int lane) {
  const uint32_t bhi = in.bhi;
  const uint64_t(&mine)[DEC_LIST] = in.mine;
  const uint32_t tau = (uint32_t)__builtin_amdgcn_readlane((int)wave_sort_desc<uint32_t>(bhi, lane), m - 1);
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < DEC_LIST; ++r) cnt += (mine[r] != 0ull && (uint32_t)(mine[r] >> 32) >= tau) ? 1 : 0;
  int total;
  const int pre = wave_excl_prefix_small(cnt, total);
  if (total <= 64) {
#pragma unroll
    for (int r = 0; r < DEC_LIST; ++r)
      if (r < cnt) surv[pre + r] = mine[r];
    __builtin_amdgcn_wave_barrier();
    const uint64_t key = sort_first_desc(lane < total ? surv[lane] : 0ull, total, lane);
    if (lane < m) top[lane] = key;
  } else {
    int ptr = 0;
    for (int r = 0; r < m; ++r) {
      uint64_t head = 0ull;
#pragma unroll
      for (int u = 0; u < DEC_LIST; ++u)
        if (u == ptr) head = mine[u];
      uint64_t best = head;
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) {
        const uint64_t o = shfl_xor_u64(best, msk);
        best = o > best ? o : best;
      }
      if (lane == 0) top[r] = best;
      if (head == best) ++ptr;  // keys are distinct: one lane advances
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// One wave: softmax attention of the query (this lane's piece qv) over the nkeys keys of the
// chunk starting at row0; writes the normalised output row to out[0..D).  A key row is
// spread over PIECES lanes, KPR rows per round.
template <typename T, int D>
__device__ __forceinline__ void wave_attend_chunk(const T* __restrict__ Kc, const T* __restrict__ Vc, int64_t row0,
                                                  int nkeys, const float (&qv)[16 / Elem<T>::bytes], float scale,
                                                  float* scw, float* out, int lane) {
  constexpr int EPP = 16 / Elem<T>::bytes;
  constexpr int PIECES = D / EPP;
  constexpr int KPR = 64 / PIECES;
  // keys and values are requested together (one memory round trip) when a row spans at most 8
  // lanes; wider rows load keys, then values, 8 rounds at a time
  constexpr int UB = PIECES < 8 ? PIECES : 8;
  constexpr bool JOINT = PIECES <= 8;
  const int piece = lane % PIECES, kl = lane / PIECES;
  int4 vraw[JOINT ? PIECES : 1];
#pragma unroll
  for (int u0 = 0; u0 < PIECES; u0 += UB) {
    int4 kraw[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int key = (u0 + u) * KPR + kl;
      const bool ok = key < nkeys;
      kraw[u] = ok ? *reinterpret_cast<const int4*>(Kc + (row0 + key) * D + piece * EPP) : make_int4(0, 0, 0, 0);
      if constexpr (JOINT)
        vraw[u] = ok ? *reinterpret_cast<const int4*>(Vc + (row0 + key) * D + piece * EPP) : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      T vals[EPP];
      __builtin_memcpy(vals, &kraw[u], 16);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPP; ++e) dot += qv[e] * Elem<T>::to_f32(vals, e);
#pragma unroll
      for (int msk = 1; msk < PIECES; msk <<= 1) dot += lane_xor(dot, msk);
      const int key = (u0 + u) * KPR + kl;
      if (piece == 0) scw[key] = key < nkeys ? scale * dot : -INFINITY;
    }
  }
  __builtin_amdgcn_wave_barrier();
  const float v = scw[lane];
  const float mx = wave_max(v);
  const float p = __expf(v - mx);
  const float sum = wave_sum(p);
  __builtin_amdgcn_wave_barrier();
  scw[lane] = p;
  __builtin_amdgcn_wave_barrier();
  float acc[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) acc[e] = 0.f;
#pragma unroll
  for (int u0 = 0; u0 < PIECES; u0 += UB) {
    int4 raw[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if constexpr (JOINT) {
        raw[u] = vraw[u0 + u];
      } else {
        const int key = (u0 + u) * KPR + kl;
        raw[u] = key < nkeys ? *reinterpret_cast<const int4*>(Vc + (row0 + key) * D + piece * EPP)
                             : make_int4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      T vals[EPP];
      __builtin_memcpy(vals, &raw[u], 16);
      const float pk = scw[(u0 + u) * KPR + kl];
#pragma unroll
      for (int e = 0; e < EPP; ++e) acc[e] += pk * Elem<T>::to_f32(vals, e);
    }
  }
#pragma unroll
  for (int msk = PIECES; msk < 64; msk <<= 1)
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] += lane_xor(acc[e], msk);
  const float inv = 1.f / sum;
  if (kl == 0) {
#pragma unroll
    for (int e = 0; e < EPP; ++e) out[piece * EPP + e] = acc[e] * inv;
  }
}

constexpr int DEC_SPLIT = 8;  // attention workgroups per head
constexpr int DEC_NWV = 16 / DEC_SPLIT;  // wavefronts per attention workgroup (16 kept slots)

// DEC_SPLIT workgroups of DEC_NWV wavefronts per head, so that the kept chunks' key and value
// reads spread over as many compute units.  In every workgroup wave 0 merges the slice lists
// and computes the fusion weights (the same result everywhere); workgroup s, wave v then
// attends to kept slot DEC_SPLIT * v + s, and workgroup 0's last wave attends to the open
// chunk meanwhile, since that needs no selection.  Each workgroup writes its weighted partial sum (its slots in
// order); decode_fuse adds the DEC_SPLIT partials.
template <typename T, int D, bool PG>
__global__ __launch_bounds__(64 * DEC_NWV) void decode_attend_kernel(const T* __restrict__ q, const T* __restrict__ qr,
                                                            const T* __restrict__ Kc,
                                                            const T* __restrict__ Vc, const T* __restrict__ Klm,
                                                            const uint64_t* __restrict__ lists,
                                                            float* __restrict__ part, int32_t* __restrict__ idx,
                                                            float* __restrict__ wout, int64_t n_in, int64_t Lmax,
                                                            int64_t Nmax, int k, float scale, DecAddr A, int mlm) {
  constexpr int EPP = 16 / Elem<T>::bytes;
  constexpr int PIECES = D / EPP;
  const int sp = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t n = dec_pos<PG>(A, bh, n_in);
  const int c = (int)(n / 64);
  const int m = min(k, c);
  const int S = (c + DEC_ROWS - 1) / DEC_ROWS;
  __shared__ uint64_t top[16];
  __shared__ uint64_t surv[64];
  __shared__ float sc_w[DEC_NWV][64];
  __shared__ float po[DEC_NWV + 1][D];
  __shared__ float wsl[17];
  const int piece = lane % PIECES;
  float qv[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) qv[e] = Elem<T>::to_f32(q, (int64_t)bh * D + piece * EPP + e);
  if (wv == 0) {
    // the slice lists are requested first; the score of the open chunk (its landmark row is
    // given) is formed meanwhile, then the selection and the weights
    MergeIn mi;
    if (m > 0) merge_load(lists + (int64_t)bh * DEC_MAX_SLICES * DEC_LIST, S, m, lane, mi);
    const int64_t own_lm = dec_lm_row<PG>(A, bh, c, Nmax) * mlm;
    float s_own = 0.f, z_own = 0.f;
    for (int u = 0; u < mlm; ++u) {
      float dot = 0.f;
      for (int e = lane; e < D; e += 64)
        dot += Elem<T>::to_f32(qr, (int64_t)bh * D + e) * Elem<T>::to_f32(Klm, (own_lm + u) * D + e);
      const float a = scale * wave_sum(dot);
      if (u == 0) {
        s_own = a;
        z_own = 1.f;
      } else if (a > s_own) {
        z_own = z_own * __expf(s_own - a) + 1.f;
        s_own = a;
      } else {
        z_own += __expf(a - s_own);
      }
    }
    if (mlm > 1) s_own += __logf(z_own);
    if (m > 0) wave_merge_lists(mi, m, top, surv, lane);
    const bool used = lane < m || lane == 16;
    const float sv = lane < m ? key_score(top[lane]) : (lane == 16 ? s_own : -INFINITY);
    const float smax = wave_max(sv);
    const float ev = used ? __expf(sv - smax) : 0.f;
    const float den = wave_sum(ev);
    if (lane < 17) wsl[lane] = ev / den;
  } else if (wv == DEC_NWV - 1 && sp == 0) {
    wave_attend_chunk<T, D>(Kc, Vc, dec_chunk_row<PG>(A, bh, c, Lmax), (int)(n - (int64_t)c * 64) + 1, qv, scale,
                            sc_w[wv], po[DEC_NWV], lane);
  }
  __syncthreads();
  const int slot = DEC_SPLIT * wv + sp;
  if (slot < m)
    wave_attend_chunk<T, D>(Kc, Vc, dec_chunk_row<PG>(A, bh, (int)key_index(top[slot]), Lmax), 64, qv, scale,
                            sc_w[wv], po[wv], lane);
  __syncthreads();
  for (int e = tid; e < D; e += 64 * DEC_NWV) {
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < DEC_NWV; ++v)
      if (DEC_SPLIT * v + sp < m) acc += wsl[DEC_SPLIT * v + sp] * po[v][e];
    if (sp == 0) acc += wsl[16] * po[DEC_NWV][e];
    part[((int64_t)bh * DEC_SPLIT + sp) * D + e] = acc;
  }
  if (sp == 0 && tid <= k) {
    const bool used = tid < m || tid == k;
    idx[(int64_t)bh * (k + 1) + tid] = tid == k ? c : (used ? key_index(top[tid]) : -1);
    wout[(int64_t)bh * (k + 1) + tid] = tid == k ? wsl[16] : (used ? wsl[tid] : 0.f);
  }
}

// o = the sum of a head's DEC_SPLIT partial outputs, in workgroup order.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_fuse_kernel(const float* __restrict__ part, T* __restrict__ o) {
  const int bh = blockIdx.x;
  for (int e = threadIdx.x; e < D; e += 64) {
    float acc = 0.f;
#pragma unroll
    for (int sp = 0; sp < DEC_SPLIT; ++sp) acc += part[((int64_t)bh * DEC_SPLIT + sp) * D + e];
    Elem<T>::store(o, (int64_t)bh * D + e, acc);
  }
}

int decode_split() { return DEC_SPLIT; }

template <typename T, int D, bool PG>
static hipError_t decode_t(const void* q, const void* qr, const void* k_new, const void* v_new, void* Kc, void* Vc,
                           const void* Klm, bool lf, int mlm, int64_t n, int64_t Lmax, int64_t Nmax, void* o,
                           int32_t* idx, float* w, int BH, int k, float scale, const DecodeBufs& ws, const DecAddr& A,
                           hipStream_t st) {
  // n: the position (contiguous caches) or the largest position of the batch (paged), which sizes the scan
  const int S = decode_slices(n);
  // the landmark scores use the retrieval query (the attention query when none is given)
  const T* qs = (const T*)(qr ? qr : q);
  if (mlm > 1)
    HILS_LAUNCH("decode_scan", (decode_scan_kernel<T, D, false, PG, true>), dim3(S > 0 ? S : 1, BH), dim3(256), 0, st,
                qs, (const T*)k_new, (const T*)v_new, (T*)Kc, (T*)Vc, (const T*)Klm, (T*)nullptr, ws.lists, n, Lmax,
                Nmax, scale, A, mlm);
  else if (lf)
    HILS_LAUNCH("decode_scan", (decode_scan_kernel<T, D, true, PG, false>), dim3(S + 1, BH), dim3(256), 0, st, qs,
                (const T*)k_new, (const T*)v_new, (T*)Kc, (T*)Vc, (const T*)Klm, (T*)Klm, ws.lists, n, Lmax, Nmax,
                scale, A, mlm);
  else
    HILS_LAUNCH("decode_scan", (decode_scan_kernel<T, D, false, PG, false>), dim3(S > 0 ? S : 1, BH), dim3(256), 0, st,
                qs,
                (const T*)k_new, (const T*)v_new, (T*)Kc, (T*)Vc, (const T*)Klm, (T*)nullptr, ws.lists, n, Lmax,
                Nmax, scale, A, mlm);
  HILS_LAUNCH("decode_attend", (decode_attend_kernel<T, D, PG>), dim3(DEC_SPLIT, BH), dim3(64 * DEC_NWV), 0, st,
              (const T*)q, qs, (const T*)Kc, (const T*)Vc, (const T*)Klm, ws.lists, ws.part, idx, w, n, Lmax, Nmax, k,
              scale, A, mlm);
  HILS_LAUNCH("decode_fuse", (decode_fuse_kernel<T, D>), dim3(BH), dim3(64), 0, st, ws.part, (T*)o);
  return hipGetLastError();
}

template <bool PG>
static hipError_t decode_dispatch(int dt, int d, const void* q, const void* qr, const void* k_new, const void* v_new,
                                  void* Kc, void* Vc, const void* Klm, bool lf, int mlm, int64_t n, int64_t Lmax,
                                  int64_t Nmax,
                                  void* o, int32_t* idx, float* w, int BH, int k, float scale, const DecodeBufs& ws,
                                  const DecAddr& A, hipStream_t st) {
  if (dt == 0)
    return d == 64 ? decode_t<bf16_t, 64, PG>(q, qr, k_new, v_new, Kc, Vc, Klm, lf, mlm, n, Lmax, Nmax, o, idx, w, BH, k,
                                              scale, ws, A, st)
                   : decode_t<bf16_t, 128, PG>(q, qr, k_new, v_new, Kc, Vc, Klm, lf, mlm, n, Lmax, Nmax, o, idx, w, BH, k,
                                               scale, ws, A, st);
  return d == 64 ? decode_t<float, 64, PG>(q, qr, k_new, v_new, Kc, Vc, Klm, lf, mlm, n, Lmax, Nmax, o, idx, w, BH, k,
                                           scale, ws, A, st)
                 : decode_t<float, 128, PG>(q, qr, k_new, v_new, Kc, Vc, Klm, lf, mlm, n, Lmax, Nmax, o, idx, w, BH, k,
                                            scale, ws, A, st);
}

hipError_t launch_decode_paged(int dt, int d, const void* q, const void* qr, const void* k_new, const void* v_new,
                               void* Kp, void* Vp, void* Klm_p, bool lf, int mlm, const int32_t* page_table, int max_pages,
                               int64_t pages, const int64_t* n_ctx, int64_t n_max, int B, int H, void* o,
                               int32_t* idx, float* w, int k, float scale, const DecodeBufs& ws, hipStream_t st) {
  const DecAddr A{page_table, n_ctx, max_pages, H, pages};
  return decode_dispatch<true>(dt, d, q, qr, k_new, v_new, Kp, Vp, Klm_p, lf, mlm, n_max, 0, 0, o, idx, w, B * H, k,
                               scale, ws, A, st);
}

hipError_t launch_decode(int dt, int d, const void* q, const void* qr, const void* k_new, const void* v_new, void* Kc,
                         void* Vc, const void* Klm, bool lf, int mlm, int64_t n, int64_t Lmax, int64_t Nmax, void* o,
                         int32_t* idx, float* w, int BH, int k, float scale, const DecodeBufs& ws, hipStream_t st) {
  const DecAddr A{nullptr, nullptr, 0, 1, 0};
  return decode_dispatch<false>(dt, d, q, qr, k_new, v_new, Kc, Vc, Klm, lf, mlm, n, Lmax, Nmax, o, idx, w, BH, k,
                                scale, ws, A, st);
}

}  // namespace hils
