// Landmark-free chunk keys: the landmark-free alternative that the HiLS summary page (ai-feeds,
// "Method" > "Input & chunking") mentions, read as: a chunk's landmark is the mean of its keys,
// and for the query's own chunk only the keys up to the query are averaged, so nothing after
// the query enters its scores.
//
//   chunk_mean  one workgroup per (chunk, head): 16-byte loads of the chunk's 64 key rows, fp32
//               sums per row group, the groups added in LDS, times 1/64 (exact), rounded to the
//               element type.  Reads the keys once (HBM-bound, 2d B per key row for bf16).
//   lf_own      one workgroup per (chunk, head), after the selection: the lanes first request their
//               query elements and kept past scores, then prefix means of the chunk's keys in LDS
//               (fp32, row segments scanned at once), the own-chunk score of each query against its
//               prefix mean (four lanes per query), and the own slot's score and the fusion
//               weights rewritten.  Reads Q (or the retrieval queries) and K once, and the
//               selection outputs once.
//   lf_bwd      the backward's tail, per (chunk, head): the mean paths into dK (reverse prefix sums
//               over the chunk's queries plus the past chunk's mean gradient / 64); the own slot's
//               score gradient against the causal means goes into dQ (or dQ_ret) in dq_reduce.
#include "hils_device.h"
#include "hils_launch.h"
#include "lf_means.h"

namespace hils {

template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_mean_kernel(const T* __restrict__ K, T* __restrict__ Klm, int64_t Lk,
                                                         int64_t Nlm) {
  constexpr int EPP = 16 / Elem<T>::bytes;  // elements per 16-byte piece
  constexpr int PIECES = D / EPP;           // pieces per row
  constexpr int G = 256 / PIECES;           // row groups
  constexpr int RPG = 64 / G;               // rows per group
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int piece = tid % PIECES, g = tid / PIECES;
  const T* base = K + ((int64_t)bh * Lk + (int64_t)j * 64) * D + piece * EPP;
  int4 raw[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i) raw[i] = *reinterpret_cast<const int4*>(base + (int64_t)(g + i * G) * D);
  float acc[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    T vals[EPP];
    __builtin_memcpy(vals, &raw[i], 16);
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] += Elem<T>::to_f32(vals, e);
  }
  __shared__ float part[G][D];
#pragma unroll
  for (int e = 0; e < EPP; ++e) part[g][piece * EPP + e] = acc[e];
  __syncthreads();
  for (int e = tid; e < D; e += 256) {
    float s = 0.f;
#pragma unroll 8
    for (int i = 0; i < G; ++i) s += part[i][e];
    Elem<T>::store(Klm, ((int64_t)bh * Nlm + j) * D + e, s * (1.f / 64.f));
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void lf_own_kernel(const T* __restrict__ Qs, const T* __restrict__ K,
                                                     const int32_t* __restrict__ idx, float* __restrict__ sel,
                                                     float* __restrict__ w, int L, int k, float scale) {
  constexpr int EPP = 16 / Elem<T>::bytes;
  constexpr int KS = D + 1;     // padded LDS row
  constexpr int EQ = D / 4;     // query elements per lane (four lanes per query)
  constexpr int SEG = 256 / D;  // row segments of the prefix scan
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int64_t row0 = (int64_t)bh * L + (int64_t)c * 64;
  const int q = tid >> 2, part = tid & 3;
  const int k1 = k + 1;
  const int64_t base = (row0 + q) * k1;
  __shared__ float km[64 * KS];
  __shared__ float segsum[SEG][D];
  // this lane's query elements and kept past slots are requested first
  int4 qraw[EQ / EPP];
#pragma unroll
  for (int v = 0; v < EQ / EPP; ++v)
    qraw[v] = *reinterpret_cast<const int4*>(Qs + (row0 + q) * D + part * EQ + v * EPP);
  int ix[4];
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = part + 4 * i;
    ix[i] = r < k ? idx[base + r] : -1;
    sv[i] = r < k ? sel[base + r] : 0.f;
  }
  stage_prefix_means<T, D>(K, row0, km, segsum, tid);
  // own-chunk score of each query, then its fusion weights
  float dot = 0.f;
#pragma unroll
  for (int v = 0; v < EQ / EPP; ++v) {
    T vals[EPP];
    __builtin_memcpy(vals, &qraw[v], 16);
#pragma unroll
    for (int e = 0; e < EPP; ++e) dot += Elem<T>::to_f32(vals, e) * km[q * KS + part * EQ + v * EPP + e];
  }
  dot += lane_xor(dot, 1);
  dot += lane_xor(dot, 2);
  const float s_own = scale * dot;
  float mx = s_own;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (ix[i] >= 0) mx = fmaxf(mx, sv[i]);
  mx = fmaxf(mx, lane_xor(mx, 1));
  mx = fmaxf(mx, lane_xor(mx, 2));
  float den = part == 0 ? __expf(s_own - mx) : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (ix[i] >= 0) den += __expf(sv[i] - mx);
  den += lane_xor(den, 1);
  den += lane_xor(den, 2);
  const float inv = 1.f / den;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = part + 4 * i;
    if (r < k) w[base + r] = ix[i] >= 0 ? __expf(sv[i] - mx) * inv : 0.f;
  }
  if (part == (k & 3)) {
    sel[base + k] = s_own;
    w[base + k] = __expf(s_own - mx) * inv;
  }
}

// Backward tail of landmark-free chunks, per (chunk c, head), after klm_bwd: each key i of the chunk
// gets scale ds_t,own qs_t / (t - 64c + 1) summed over the chunk's queries t >= i (a reverse prefix
// sum over t), plus dKlm_c / 64 for the past chunks' use of its mean (dKlm_c from klm_bwd, past pairs
// only).  The own slot's dQs term, scale ds_t,own m_t, is added by dq_reduce.  The rounding of the means
// is passed straight through.  dK is read, added to and written.
template <typename T, int D>
__global__ __launch_bounds__(256) void lf_bwd_kernel(const T* __restrict__ Qs, const float* __restrict__ ds,
                                                     const float* __restrict__ dKlm, float* __restrict__ dK, int L,
                                                     int N, int k, float scale) {
  constexpr int EPP = 16 / Elem<T>::bytes;
  constexpr int KS = D + 1;
  constexpr int EQ = D / 4;
  constexpr int SEG = 256 / D;
  constexpr int RS = 64 / SEG;
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int64_t row0 = (int64_t)bh * L + (int64_t)c * 64;
  const int q = tid >> 2, part = tid & 3;
  __shared__ float gm[64 * KS];
  __shared__ float segsum[SEG][D];
  int4 qraw[EQ / EPP];
#pragma unroll
  for (int v = 0; v < EQ / EPP; ++v)
    qraw[v] = *reinterpret_cast<const int4*>(Qs + (row0 + q) * D + part * EQ + v * EPP);
  const float sds = scale * ds[(row0 + q) * (k + 1) + k];
  const float e_off = dKlm[((int64_t)bh * N + c) * D + tid % D] * (1.f / 64.f);
  // g_t = scale ds_t qs_t / (t + 1)
  {
    const float inv_cnt = 1.f / (float)(q + 1);
#pragma unroll
    for (int v = 0; v < EQ / EPP; ++v) {
      T vals[EPP];
      __builtin_memcpy(vals, &qraw[v], 16);
#pragma unroll
      for (int e = 0; e < EPP; ++e) gm[q * KS + part * EQ + v * EPP + e] = sds * Elem<T>::to_f32(vals, e) * inv_cnt;
    }
  }
  __syncthreads();
  // key i receives sum over t >= i of g_t: reverse prefix sums in SEG row segments, offset by the later ones
  const int e = tid % D, sg = tid / D;
  float run = 0.f;
#pragma unroll
  for (int i = RS - 1; i >= 0; --i) {
    const int r = sg * RS + i;
    run += gm[r * KS + e];
    gm[r * KS + e] = run;
  }
  segsum[sg][e] = run;
  __syncthreads();
  float off = e_off;
  for (int j = sg + 1; j < SEG; ++j) off += segsum[j][e];
#pragma unroll
  for (int i = 0; i < RS; ++i) {
    const int r = sg * RS + i;
    dK[(row0 + r) * D + e] += gm[r * KS + e] + off;
  }
}

template <typename T, int D>
static hipError_t lf_bwd_t(const void* Qs, const float* ds, const float* dKlm, float* dK, int BH, int L, int N, int k,
                           float scale, hipStream_t st) {
  HILS_LAUNCH("lf_bwd", (lf_bwd_kernel<T, D>), dim3(N, BH), dim3(256), 0, st, (const T*)Qs, ds, dKlm, dK, L, N, k,
              scale);
  return hipGetLastError();
}

hipError_t launch_lf_bwd(int dt, int d, const void* Qs, const float* ds, const float* dKlm, float* dK, int BH, int L,
                         int N, int k, float scale, hipStream_t st) {
  if (dt == 0)
    return d == 64 ? lf_bwd_t<bf16_t, 64>(Qs, ds, dKlm, dK, BH, L, N, k, scale, st)
                   : lf_bwd_t<bf16_t, 128>(Qs, ds, dKlm, dK, BH, L, N, k, scale, st);
  return d == 64 ? lf_bwd_t<float, 64>(Qs, ds, dKlm, dK, BH, L, N, k, scale, st)
                 : lf_bwd_t<float, 128>(Qs, ds, dKlm, dK, BH, L, N, k, scale, st);
}

template <typename T, int D>
static hipError_t chunk_means_t(const void* K, void* Klm, int BH, int64_t Lk, int64_t Nlm, int nchunks,
                                hipStream_t st) {
  if (nchunks <= 0) return hipSuccess;
  HILS_LAUNCH("chunk_mean", (chunk_mean_kernel<T, D>), dim3(nchunks, BH), dim3(256), 0, st, (const T*)K, (T*)Klm,
              Lk, Nlm);
  return hipGetLastError();
}

hipError_t launch_chunk_means(int dt, int d, const void* K, void* Klm, int BH, int64_t Lk, int64_t Nlm, int nchunks,
                              hipStream_t st) {
  if (dt == 0)
    return d == 64 ? chunk_means_t<bf16_t, 64>(K, Klm, BH, Lk, Nlm, nchunks, st)
                   : chunk_means_t<bf16_t, 128>(K, Klm, BH, Lk, Nlm, nchunks, st);
  return d == 64 ? chunk_means_t<float, 64>(K, Klm, BH, Lk, Nlm, nchunks, st)
                 : chunk_means_t<float, 128>(K, Klm, BH, Lk, Nlm, nchunks, st);
}

template <typename T, int D>
static hipError_t lf_own_t(const void* Qs, const void* K, const int32_t* idx, float* sel, float* w, int BH, int L,
                           int k, float scale, hipStream_t st) {
  HILS_LAUNCH("lf_own", (lf_own_kernel<T, D>), dim3(L / 64, BH), dim3(256), 0, st, (const T*)Qs, (const T*)K, idx,
              sel, w, L, k, scale);
  return hipGetLastError();
}

hipError_t launch_lf_own(int dt, int d, const void* Qs, const void* K, const int32_t* idx, float* sel, float* w,
                         int BH, int L, int k, float scale, hipStream_t st) {
  if (dt == 0)
    return d == 64 ? lf_own_t<bf16_t, 64>(Qs, K, idx, sel, w, BH, L, k, scale, st)
                   : lf_own_t<bf16_t, 128>(Qs, K, idx, sel, w, BH, L, k, scale, st);
  return d == 64 ? lf_own_t<float, 64>(Qs, K, idx, sel, w, BH, L, k, scale, st)
                 : lf_own_t<float, 128>(Qs, K, idx, sel, w, BH, L, k, scale, st);
}

}  // namespace hils
