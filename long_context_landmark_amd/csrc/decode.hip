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
// them), so the scan is spread over many workgroups with 16-byte coalesced
// loads and dot products on VALU; each slice keeps its local top-16 as sorted
// 64-bit keys.  The second kernel runs one workgroup per kept chunk (split-K
// over the k+1 chunks of the query): each merges the slice lists (the same
// result in every workgroup), attends to its chunk and publishes its weighted
// partial; the last workgroup of the head to finish sums the partials in slot
// order and writes o, idx and w.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

constexpr int DEC_SLICE = 128;  // landmark rows per scan workgroup

int decode_slices(int64_t n_ctx) { return (int)((n_ctx / 64 + DEC_SLICE - 1) / DEC_SLICE); }

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_scan_kernel(const T* __restrict__ q, const T* __restrict__ k_new,
                                                          const T* __restrict__ v_new, T* __restrict__ Kc,
                                                          T* __restrict__ Vc, const T* __restrict__ Klm,
                                                          uint64_t* __restrict__ cand, int* __restrict__ ticket,
                                                          int64_t n, int64_t Lmax, int64_t Nmax, int S, float scale) {
  constexpr int EPP = 16 / Elem<T>::bytes;  // elements per 16-byte piece
  constexpr int PIECES = D / EPP;           // pieces per row
  constexpr int RPR = 256 / PIECES;         // rows per round
  const int s = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int c = (int)(n / 64);
  if (s == 0) {
    // append the new key and value (idempotent) and reset the head's arrival counter
    for (int e = tid; e < D; e += 256) {
      Kc[((int64_t)bh * Lmax + n) * D + e] = k_new[(int64_t)bh * D + e];
      Vc[((int64_t)bh * Lmax + n) * D + e] = v_new[(int64_t)bh * D + e];
    }
    if (tid == 0) ticket[bh] = 0;
  }
  const int j0 = s * DEC_SLICE;
  if (j0 >= c) return;
  const int j1 = min(c, j0 + DEC_SLICE);
  __shared__ uint64_t keys[DEC_SLICE];
  const int piece = tid % PIECES, rr = tid / PIECES;
  float qv[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) qv[e] = Elem<T>::to_f32(q, (int64_t)bh * D + piece * EPP + e);
  const T* base = Klm + (int64_t)bh * Nmax * D;
#pragma unroll
  for (int round = 0; round < DEC_SLICE / RPR; ++round) {
    const int j = j0 + round * RPR + rr;
    float dot = 0.f;
    if (j < j1) {
      T vals[EPP];
      const int4 raw = *reinterpret_cast<const int4*>(base + (int64_t)j * D + piece * EPP);
      __builtin_memcpy(vals, &raw, 16);
#pragma unroll
      for (int e = 0; e < EPP; ++e) dot += qv[e] * Elem<T>::to_f32(vals, e);
    }
#pragma unroll
    for (int m = 1; m < PIECES; m <<= 1) dot += __shfl_xor(dot, m);
    if (piece == 0) keys[round * RPR + rr] = (j < j1) ? make_key(scale * dot, j) : 0ull;
  }
  __syncthreads();
  if (tid < DEC_SLICE / 16) {  // 8 lanes, 16 keys each -> one sorted top-16
    uint64_t v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = keys[tid * 16 + e];
    sort16_desc(v);
    merge16_with_lane(v, 1);
    merge16_with_lane(v, 2);
    merge16_with_lane(v, 4);
    if (tid == 0) {
      uint64_t* dst = cand + ((int64_t)bh * S + s) * 16;
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[e] = v[e];
    }
  }
}

// Merge the sorted lists b into a (both descending, 16 each): a = top-16 of the union.
__device__ __forceinline__ void merge16_local(uint64_t (&a)[16], const uint64_t (&b)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = a[i] > b[15 - i] ? a[i] : b[15 - i];
  bitonic_merge16_desc(a);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_attend_kernel(const T* __restrict__ q, const T* __restrict__ Kc,
                                                            const T* __restrict__ Vc, const T* __restrict__ Klm,
                                                            const uint64_t* __restrict__ cand,
                                                            float* __restrict__ part, int* __restrict__ ticket,
                                                            T* __restrict__ o, int32_t* __restrict__ idx,
                                                            float* __restrict__ wout, int64_t n, int64_t Lmax,
                                                            int64_t Nmax, int S, int k, float scale) {
  const int r = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = (int)(n / 64);
  const int m = min(k, c);
  if (r >= m && r != k) return;
  __shared__ uint64_t top[16];
  __shared__ float sc[64];
  __shared__ float red[4][D];
  __shared__ float s_own_s;
  __shared__ int last_s;
  // global top-m: wave 0 merges the slice lists (lane l takes lists l, l+64, ...)
  if (wv == 0) {
    uint64_t a[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) a[e] = 0ull;
    for (int s = lane; s < S; s += 64) {
      uint64_t b[16];
      const uint64_t* src = cand + ((int64_t)bh * S + s) * 16;
#pragma unroll
      for (int e = 0; e < 16; ++e) b[e] = src[e];
      merge16_local(a, b);
    }
    if (S > 1) {
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) merge16_with_lane(a, msk);
    }
    if (lane == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) top[e] = a[e];
    }
  }
  // own-chunk score (wave 1): scale * <q, Klm_c>
  if (wv == 1) {
    float dot = 0.f;
    for (int e = lane; e < D; e += 64)
      dot += Elem<T>::to_f32(q, (int64_t)bh * D + e) * Elem<T>::to_f32(Klm, ((int64_t)bh * Nmax + c) * D + e);
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) dot += __shfl_xor(dot, msk);
    if (lane == 0) s_own_s = scale * dot;
  }
  __syncthreads();
  const int j = (r == k) ? c : key_index(top[r]);
  const int nkeys = (r == k) ? (int)(n - (int64_t)c * 64) + 1 : 64;
  const int64_t row0 = (int64_t)bh * Lmax + (int64_t)j * 64;
  // scores of the chunk's keys: 4 lanes per key
  {
    const int key = tid >> 2, part_ = tid & 3;
    float dot = 0.f;
    if (key < nkeys) {
      for (int e = part_ * (D / 4); e < (part_ + 1) * (D / 4); ++e)
        dot += Elem<T>::to_f32(q, (int64_t)bh * D + e) * Elem<T>::to_f32(Kc, (row0 + key) * D + e);
    }
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    if (part_ == 0) sc[key] = key < nkeys ? scale * dot : -INFINITY;
  }
  __syncthreads();
  float mx = -INFINITY, sum = 0.f;
  {
    const float v = sc[lane];
    mx = v;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk));
    const float p = __expf(v - mx);
    sum = p;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) sum += __shfl_xor(sum, msk);
  }
  __syncthreads();
  if (wv == 0) sc[lane] = __expf(sc[lane] - mx);
  __syncthreads();
  // P V: wave wv takes keys 16wv .. 16wv+15, lane-strided over d
  for (int e = lane; e < D; e += 64) {
    float acc = 0.f;
    for (int key = 16 * wv; key < min(nkeys, 16 * wv + 16); ++key)
      acc += sc[key] * Elem<T>::to_f32(Vc, (row0 + key) * D + e);
    red[wv][e] = acc;
  }
  __syncthreads();
  // fusion weight of this slot
  float smax = s_own_s;
  for (int i = 0; i < m; ++i) smax = fmaxf(smax, key_score(top[i]));
  float den = __expf(s_own_s - smax);
  for (int i = 0; i < m; ++i) den += __expf(key_score(top[i]) - smax);
  const float s_r = (r == k) ? s_own_s : key_score(top[r]);
  const float w_r = __expf(s_r - smax) / den;
  float* dst = part + ((int64_t)bh * (k + 1) + r) * D;
  for (int e = tid; e < D; e += 256) dst[e] = w_r * (red[0][e] + red[1][e] + red[2][e] + red[3][e]) / sum;
  // last arriving workgroup of the head combines the partials in slot order
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    last_s = atomicAdd(&ticket[bh], 1) == m;
    __threadfence();
  }
  __syncthreads();
  if (!last_s) return;
  __threadfence();
  for (int e = tid; e < D; e += 256) {
    float acc = 0.f;
    for (int i = 0; i < m; ++i) acc += __builtin_nontemporal_load(part + ((int64_t)bh * (k + 1) + i) * D + e);
    acc += __builtin_nontemporal_load(part + ((int64_t)bh * (k + 1) + k) * D + e);
    Elem<T>::store(o, (int64_t)bh * D + e, acc);
  }
  if (tid <= k) {
    const bool used = tid < m || tid == k;
    const float s_t = tid == k ? s_own_s : (used ? key_score(top[tid]) : 0.f);
    idx[(int64_t)bh * (k + 1) + tid] = tid == k ? c : (used ? key_index(top[tid]) : -1);
    wout[(int64_t)bh * (k + 1) + tid] = used ? __expf(s_t - smax) / den : 0.f;
  }
  if (tid == 0) ticket[bh] = 0;
}

template <typename T, int D>
static hipError_t decode_t(const void* q, const void* k_new, const void* v_new, void* Kc, void* Vc, const void* Klm,
                           int64_t n, int64_t Lmax, int64_t Nmax, void* o, int32_t* idx, float* w, int BH, int k,
                           float scale, const DecodeBufs& ws, hipStream_t st) {
  const int S = decode_slices(n);
  hipLaunchKernelGGL((decode_scan_kernel<T, D>), dim3(S > 0 ? S : 1, BH), dim3(256), 0, st, (const T*)q,
                     (const T*)k_new, (const T*)v_new, (T*)Kc, (T*)Vc, (const T*)Klm, ws.cand, ws.ticket, n, Lmax,
                     Nmax, S, scale);
  hipLaunchKernelGGL((decode_attend_kernel<T, D>), dim3(k + 1, BH), dim3(256), 0, st, (const T*)q, (const T*)Kc,
                     (const T*)Vc, (const T*)Klm, ws.cand, ws.part, ws.ticket, (T*)o, idx, w, n, Lmax, Nmax, S, k,
                     scale);
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
