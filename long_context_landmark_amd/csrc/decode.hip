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
// workgroups and writes one fp32 score per chunk (4 bytes per 128-256 bytes
// read).  decode_attend runs one 1024-thread workgroup per head.  One wavefront
// selects the top-m from the score row: the m-th largest of the 64 lane maxima
// (a wave-wide bitonic sort) bounds the m-th largest score from below, and the
// few scores at or above it are compacted with ballots and sorted exactly.  The
// k+1 kept chunks are then split over the 16 wavefronts (split-K), each reading
// its chunk's keys and values with 16-byte loads, and the weighted per-chunk
// outputs are fused in LDS in slot order.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

constexpr int DEC_ROWS = 256;  // landmark rows per scan workgroup
constexpr int DEC_MAX_CHUNKS = 16384;  // the library's chunk limit

int decode_slices(int64_t n_ctx) { return (int)((n_ctx / 64 + DEC_ROWS - 1) / DEC_ROWS); }

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_scan_kernel(const T* __restrict__ q, const T* __restrict__ k_new,
                                                          const T* __restrict__ v_new, T* __restrict__ Kc,
                                                          T* __restrict__ Vc, const T* __restrict__ Klm,
                                                          float* __restrict__ scores, int64_t n, int64_t Lmax,
                                                          int64_t Nmax, float scale) {
  constexpr int EPP = 16 / Elem<T>::bytes;  // elements per 16-byte piece
  constexpr int PIECES = D / EPP;           // pieces per row
  constexpr int RPR = 256 / PIECES;         // rows per round
  constexpr int ROUNDS = DEC_ROWS / RPR;
  const int s = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int c = (int)(n / 64);
  if (s == 0) {
    // append the new key and value (idempotent)
    for (int e = tid; e < D; e += 256) {
      Kc[((int64_t)bh * Lmax + n) * D + e] = k_new[(int64_t)bh * D + e];
      Vc[((int64_t)bh * Lmax + n) * D + e] = v_new[(int64_t)bh * D + e];
    }
  }
  const int j0 = s * DEC_ROWS;
  if (j0 >= c) return;
  const int piece = tid % PIECES, rr = tid / PIECES;
  float qv[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) qv[e] = Elem<T>::to_f32(q, (int64_t)bh * D + piece * EPP + e);
  const T* base = Klm + (int64_t)bh * Nmax * D + piece * EPP;
  int4 raw[ROUNDS];
#pragma unroll
  for (int round = 0; round < ROUNDS; ++round) {
    const int j = j0 + round * RPR + rr;
    raw[round] = j < c ? *reinterpret_cast<const int4*>(base + (int64_t)j * D) : make_int4(0, 0, 0, 0);
  }
  float* out = scores + (int64_t)bh * Nmax;
#pragma unroll
  for (int round = 0; round < ROUNDS; ++round) {
    T vals[EPP];
    __builtin_memcpy(vals, &raw[round], 16);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < EPP; ++e) dot += qv[e] * Elem<T>::to_f32(vals, e);
#pragma unroll
    for (int m = 1; m < PIECES; m <<= 1) dot += __shfl_xor(dot, m);
    const int j = j0 + round * RPR + rr;
    if (piece == 0 && j < c) out[j] = scale * dot;
  }
}

// Wave-wide bitonic sort, descending: afterwards lane i holds the i-th largest value.
template <typename K> __device__ __forceinline__ K wave_sort_desc(K v, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const K o = shfl_xor_any(v, stride);
      const bool desc = (lane & size) == 0;
      const bool lower = (lane & stride) == 0;
      const K hi = v > o ? v : o, lo = v > o ? o : v;
      v = (desc == lower) ? hi : lo;
    }
  }
  return v;
}

// top[0..m-1] = the m best keys of sc[0..c) (score desc, index asc); sc is in LDS.  Run by one full wave.
__device__ void wave_select_topm(const float* sc, int c, int m, uint64_t* top, uint64_t* surv, int lane) {
  float mx = -INFINITY;
#pragma unroll 8
  for (int j = lane; j < c; j += 64) mx = fmaxf(mx, sc[j]);
  const float sorted = wave_sort_desc(mx, lane);
  const float tau = __shfl(sorted, m - 1);  // lane maxima are distinct candidates: tau <= m-th best
  const uint64_t below = (1ull << lane) - 1ull;
  int cnt = 0;
  for (int j0 = 0; j0 < c; j0 += 64) {
    const int j = j0 + lane;
    const float s = j < c ? sc[j] : -INFINITY;
    const bool keep = j < c && s >= tau;
    const uint64_t mask = __ballot(keep);
    if (mask) {
      const int pos = cnt + __popcll(mask & below);
      if (keep && pos < 64) surv[pos] = make_key(s, j);
      cnt += __popcll(mask);
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (cnt <= 64) {
    const uint64_t key = wave_sort_desc<uint64_t>(lane < cnt ? surv[lane] : (uint64_t)0, lane);
    if (lane < m) top[lane] = key;
  } else {
    // many exact ties at the bound: m passes of "largest key below the previous one"
    uint64_t prev = ~0ull;
    for (int r = 0; r < m; ++r) {
      uint64_t best = 0ull;
      for (int j = lane; j < c; j += 64) {
        const uint64_t key = make_key(sc[j], j);
        if (key < prev && key > best) best = key;
      }
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) {
        const uint64_t o = shfl_xor_u64(best, msk);
        best = o > best ? o : best;
      }
      if (lane == 0) top[r] = best;
      prev = best;
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// One 1024-thread workgroup per head: wave 0 selects, then each of the 16 wavefronts
// attends to one kept chunk (wave 0 also to a 17th), and the weighted per-chunk
// outputs are fused in LDS in slot order.  No cross-workgroup communication.
template <typename T, int D>
__global__ __launch_bounds__(1024) void decode_attend_kernel(const T* __restrict__ q, const T* __restrict__ Kc,
                                                             const T* __restrict__ Vc, const T* __restrict__ Klm,
                                                             const float* __restrict__ scores, T* __restrict__ o,
                                                             int32_t* __restrict__ idx, float* __restrict__ wout,
                                                             int64_t n, int64_t Lmax, int64_t Nmax, int k,
                                                             float scale) {
  constexpr int EPP = 16 / Elem<T>::bytes;
  constexpr int PIECES = D / EPP;   // 16-byte pieces per row (8 or 16 for bf16)
  constexpr int KPR = 64 / PIECES;  // keys per round when a row is spread over PIECES lanes
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = (int)(n / 64);
  const int m = min(k, c);
  __shared__ float all_s[DEC_MAX_CHUNKS];
  __shared__ uint64_t top[16];
  __shared__ uint64_t surv[64];
  __shared__ float qs[D];
  __shared__ float sc_w[16][64];
  __shared__ float po[17][D];
  __shared__ float s_own_s;
  for (int e = tid; e < D; e += 1024) qs[e] = Elem<T>::to_f32(q, (int64_t)bh * D + e);
  if (m > 0) {
    const float* srow = scores + (int64_t)bh * Nmax;
#pragma unroll 8
    for (int jj = tid; jj < c; jj += 1024) all_s[jj] = srow[jj];
  }
  __syncthreads();
  if (wv == 0 && m > 0) wave_select_topm(all_s, c, m, top, surv, lane);
  if (wv == 1) {
    float dot = 0.f;
    for (int e = lane; e < D; e += 64) dot += qs[e] * Elem<T>::to_f32(Klm, ((int64_t)bh * Nmax + c) * D + e);
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) dot += __shfl_xor(dot, msk);
    if (lane == 0) s_own_s = scale * dot;
  }
  __syncthreads();
  float smax = s_own_s;
  for (int i = 0; i < m; ++i) smax = fmaxf(smax, key_score(top[i]));
  float den = __expf(s_own_s - smax);
  for (int i = 0; i < m; ++i) den += __expf(key_score(top[i]) - smax);
  const int piece = lane % PIECES, kl = lane / PIECES;
  for (int item = wv; item <= m; item += 16) {
    const int r = item < m ? item : k;
    const int j = item < m ? key_index(top[item]) : c;
    const int nkeys = item < m ? 64 : (int)(n - (int64_t)c * 64) + 1;
    const int64_t row0 = (int64_t)bh * Lmax + (int64_t)j * 64;
    // logits: a row spread over PIECES lanes, KPR rows per round, loads issued 8 rounds at a time
    constexpr int UB = PIECES < 8 ? PIECES : 8;
#pragma unroll
    for (int u0 = 0; u0 < PIECES; u0 += UB) {
      int4 raw[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int key = (u0 + u) * KPR + kl;
        raw[u] = key < nkeys ? *reinterpret_cast<const int4*>(Kc + (row0 + key) * D + piece * EPP)
                             : make_int4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        T vals[EPP];
        __builtin_memcpy(vals, &raw[u], 16);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPP; ++e) dot += qs[piece * EPP + e] * Elem<T>::to_f32(vals, e);
#pragma unroll
        for (int msk = 1; msk < PIECES; msk <<= 1) dot += __shfl_xor(dot, msk);
        const int key = (u0 + u) * KPR + kl;
        if (piece == 0) sc_w[wv][key] = key < nkeys ? scale * dot : -INFINITY;
      }
    }
    __builtin_amdgcn_wave_barrier();
    const float v = sc_w[wv][lane];
    float mx = v;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk));
    const float p = __expf(v - mx);
    float sum = p;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) sum += __shfl_xor(sum, msk);
    __builtin_amdgcn_wave_barrier();
    sc_w[wv][lane] = p;
    __builtin_amdgcn_wave_barrier();
    // P V with the same lane layout: rows u*KPR + kl, elements piece*EPP ..
    float acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u0 = 0; u0 < PIECES; u0 += UB) {
      int4 raw[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int key = (u0 + u) * KPR + kl;
        raw[u] = key < nkeys ? *reinterpret_cast<const int4*>(Vc + (row0 + key) * D + piece * EPP)
                             : make_int4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        T vals[EPP];
        __builtin_memcpy(vals, &raw[u], 16);
        const float pk = sc_w[wv][(u0 + u) * KPR + kl];
#pragma unroll
        for (int e = 0; e < EPP; ++e) acc[e] += pk * Elem<T>::to_f32(vals, e);
      }
    }
#pragma unroll
    for (int msk = PIECES; msk < 64; msk <<= 1)
#pragma unroll
      for (int e = 0; e < EPP; ++e) acc[e] += __shfl_xor(acc[e], msk);
    const float s_r = item < m ? key_score(top[item]) : s_own_s;
    const float f = __expf(s_r - smax) / den / sum;
    const int slot = item < m ? item : 16;
    if (kl == 0) {
#pragma unroll
      for (int e = 0; e < EPP; ++e) po[slot][piece * EPP + e] = f * acc[e];
    }
    (void)r;
  }
  __syncthreads();
  for (int e = tid; e < D; e += 1024) {
    float acc = 0.f;
    for (int i = 0; i < m; ++i) acc += po[i][e];
    acc += po[16][e];
    Elem<T>::store(o, (int64_t)bh * D + e, acc);
  }
  if (tid <= k) {
    const bool used = tid < m || tid == k;
    const float s_t = tid == k ? s_own_s : (used ? key_score(top[tid]) : 0.f);
    idx[(int64_t)bh * (k + 1) + tid] = tid == k ? c : (used ? key_index(top[tid]) : -1);
    wout[(int64_t)bh * (k + 1) + tid] = used ? __expf(s_t - smax) / den : 0.f;
  }
}

template <typename T, int D>
static hipError_t decode_t(const void* q, const void* k_new, const void* v_new, void* Kc, void* Vc, const void* Klm,
                           int64_t n, int64_t Lmax, int64_t Nmax, void* o, int32_t* idx, float* w, int BH, int k,
                           float scale, const DecodeBufs& ws, hipStream_t st) {
  const int S = decode_slices(n);
  HILS_LAUNCH("decode_scan", (decode_scan_kernel<T, D>), dim3(S > 0 ? S : 1, BH), dim3(256), 0, st, (const T*)q,
              (const T*)k_new, (const T*)v_new, (T*)Kc, (T*)Vc, (const T*)Klm, ws.scores, n, Lmax, Nmax, scale);
  HILS_LAUNCH("decode_attend", (decode_attend_kernel<T, D>), dim3(BH), dim3(1024), 0, st, (const T*)q, (const T*)Kc,
              (const T*)Vc, (const T*)Klm, ws.scores, (T*)o, idx, w, n, Lmax, Nmax, k, scale);
  return hipGetLastError();
}

hipError_t launch_decode(int dt, int d, const void* q, const void* k_new, const void* v_new, void* Kc, void* Vc,
                         const void* Klm, int64_t n, int64_t Lmax, int64_t Nmax, void* o, int32_t* idx, float* w,
                         int BH, int k, float scale, const DecodeBufs& ws, hipStream_t st) {
  if (dt == 0)
    return d == 64 ? decode_t<bf16_t, 64>(q, k_new, v_new, Kc, Vc, Klm, n, Lmax, Nmax, o, idx, w, BH, k, scale, ws, st)
                   : decode_t<bf16_t, 128>(q, k_new, v_new, Kc, Vc, Klm, n, Lmax, Nmax, o, idx, w, BH, k, scale, ws,
                                           st);
  return d == 64 ? decode_t<float, 64>(q, k_new, v_new, Kc, Vc, Klm, n, Lmax, Nmax, o, idx, w, BH, k, scale, ws, st)
                 : decode_t<float, 128>(q, k_new, v_new, Kc, Vc, Klm, n, Lmax, Nmax, o, idx, w, BH, k, scale, ws, st);
}

}  // namespace hils
