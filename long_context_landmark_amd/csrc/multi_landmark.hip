// Several landmarks per chunk: the HiLS summary page (ai-feeds, "Method" > "Input & chunking")
// gives a chunk a few landmarks (usually its first and last token) and "Key modules" item 1 a
// softmax over a chunk's landmark scores before the chunk-level one.  Read as: the chunk score is
// the log-sum-exp of the chunk's m landmark scores.  K_lm is [B][H][N][m][d].
//
//   ml_scores   one workgroup per (query chunk, head): the 64 queries staged as fp32 in LDS; for
//               every tile of 64 chunks up to the query chunk and every landmark, the landmark
//               rows staged and the 64 x 64 dot products formed on the VALU (lane = query, wave =
//               16 chunks, so landmark reads are LDS broadcasts), folded into a running
//               log-sum-exp per (query, chunk).  Writes the causal chunk scores S [BH][L][N] (fp32).
//   ml_select   one wave per query row: the m = min(k, c) best past chunks by (score desc, index
//               asc) in k rounds of a wave maximum over 64-bit keys, the own chunk's score, and
//               the fusion weights; or, for a caller-given selection, its scores and weights.
// The selection outputs then feed the routing and chunk-attention kernels of the plain forward.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

template <typename T, int D>
__global__ __launch_bounds__(256) void ml_scores_kernel(const T* __restrict__ Qs, const T* __restrict__ Klm,
                                                        float* __restrict__ S, int L, int N, int m, float scale) {
  constexpr int EPP = 16 / Elem<T>::bytes;
  constexpr int PIECES = D / EPP;
  constexpr int RPR = 256 / PIECES;
  constexpr int KS = D + 1;
  const int qc = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int q = tid & 63, jg = tid >> 6;  // lane: query; wave: 16 chunks of the tile
  const int64_t row0 = (int64_t)bh * L + (int64_t)qc * 64;
  __shared__ float qs[64 * KS];
  __shared__ float lm[64 * KS];
  const int piece = tid % PIECES, rr = tid / PIECES;
#pragma unroll
  for (int r0 = 0; r0 < 64; r0 += RPR) {
    const int r = r0 + rr;
    const int4 raw = *reinterpret_cast<const int4*>(Qs + (row0 + r) * D + piece * EPP);
    T vals[EPP];
    __builtin_memcpy(vals, &raw, 16);
#pragma unroll
    for (int e = 0; e < EPP; ++e) qs[r * KS + piece * EPP + e] = Elem<T>::to_f32(vals, e);
  }
  for (int j0 = 0; j0 <= qc; j0 += 64) {
    float mx[16], z[16];
    for (int u = 0; u < m; ++u) {
      __syncthreads();  // the previous landmark tile is consumed
#pragma unroll
      for (int r0 = 0; r0 < 64; r0 += RPR) {
        const int jj = r0 + rr, j = j0 + jj;
        int4 raw = make_int4(0, 0, 0, 0);
        if (j <= qc) raw = *reinterpret_cast<const int4*>(Klm + (((int64_t)bh * N + j) * m + u) * D + piece * EPP);
        T vals[EPP];
        __builtin_memcpy(vals, &raw, 16);
#pragma unroll
        for (int e = 0; e < EPP; ++e) lm[jj * KS + piece * EPP + e] = Elem<T>::to_f32(vals, e);
      }
      __syncthreads();
      float acc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      for (int e = 0; e < D; ++e) {
        const float qv = qs[q * KS + e];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += qv * lm[(jg * 16 + i) * KS + e];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = scale * acc[i];
        if (u == 0) {
          mx[i] = a;
          z[i] = 1.f;
        } else if (a > mx[i]) {
          z[i] = z[i] * __expf(mx[i] - a) + 1.f;
          mx[i] = a;
        } else {
          z[i] += __expf(a - mx[i]);
        }
      }
    }
    float* srow = S + (row0 + q) * N;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + jg * 16 + i;
      if (j <= qc) srow[j] = m == 1 ? mx[i] : mx[i] + __logf(z[i]);
    }
  }
}

__global__ __launch_bounds__(256) void ml_select_kernel(const float* __restrict__ S, int32_t* __restrict__ idx,
                                                        float* __restrict__ sel, float* __restrict__ w, int64_t rows,
                                                        int L, int N, int k, int select) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int t = (int)(row % L);
  const int c = t / 64;
  const int m = min(k, c);
  const int k1 = k + 1;
  const float* srow = S + row * N;
  const int64_t base = row * k1;
  // this lane's slot: a kept past chunk (lane < k) or the own chunk (lane == k)
  int ix = -1;
  float sv = -INFINITY;
  if (select) {
    uint64_t prev = ~0ull;
    for (int r = 0; r < m; ++r) {
      uint64_t best = 0ull;
      for (int j = lane; j < c; j += 64) {
        const uint64_t key = make_key(srow[j], j);
        if (key < prev && key > best) best = key;
      }
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) {
        const uint64_t o = shfl_xor_u64(best, msk);
        best = o > best ? o : best;
      }
      if (lane == r) {
        ix = key_index(best);
        sv = key_score(best);
      }
      prev = best;
    }
  } else if (lane < k) {
    ix = idx[base + lane];
    if (ix >= 0) sv = srow[ix];
  }
  if (lane == k) {
    ix = c;
    sv = srow[c];
  }
  const bool used = lane <= k && ix >= 0;
  const float smax = wave_max(used ? sv : -INFINITY);
  const float ev = used ? __expf(sv - smax) : 0.f;
  const float den = wave_sum(ev);
  if (lane <= k) {
    if (select) idx[base + lane] = ix;
    sel[base + lane] = used ? sv : -INFINITY;
    if (w) w[base + lane] = ev / den;
  }
}

template <typename T, int D>
static hipError_t ml_scores_t(const void* Qs, const void* Klm, float* S, int BH, int L, int N, int m, float scale,
                              hipStream_t st) {
  HILS_LAUNCH("ml_scores", (ml_scores_kernel<T, D>), dim3(L / 64, BH), dim3(256), 0, st, (const T*)Qs,
              (const T*)Klm, S, L, N, m, scale);
  return hipGetLastError();
}

hipError_t launch_ml_selection(int dt, int d, const void* Qs, const void* Klm, int m, float* S, int32_t* idx,
                               float* sel, float* w, int BH, int L, int N, int k, int select, float scale,
                               hipStream_t st) {
  hipError_t e;
  if (dt == 0)
    e = d == 64 ? ml_scores_t<bf16_t, 64>(Qs, Klm, S, BH, L, N, m, scale, st)
                : ml_scores_t<bf16_t, 128>(Qs, Klm, S, BH, L, N, m, scale, st);
  else
    e = d == 64 ? ml_scores_t<float, 64>(Qs, Klm, S, BH, L, N, m, scale, st)
                : ml_scores_t<float, 128>(Qs, Klm, S, BH, L, N, m, scale, st);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)BH * L;
  HILS_LAUNCH("ml_select", ml_select_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, S, idx, sel, w,
              rows, L, N, k, select);
  return hipGetLastError();
}

}  // namespace hils
