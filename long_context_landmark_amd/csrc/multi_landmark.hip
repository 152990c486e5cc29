// Several landmarks per chunk: the HiLS summary page (ai-feeds, "Method" > "Input & chunking")
// gives a chunk a few landmarks (usually its first and last token) and "Key modules" item 1 a
// softmax over a chunk's landmark scores before the chunk-level one.  Read as: the chunk score is
// the log-sum-exp of the chunk's m landmark scores.  K_lm is [B][H][N][m][d].
//
// A selection (select = 1) runs in the selection kernel of scores_topk.hip, which forms the
// log-sum-exp scores from every landmark's MFMA products itself (no score matrix).  For a
// caller-given selection, ml_fixed_selection scores just the k + 1 given chunks of each query
// row: one thread per row, fp32 dot products, the log-sum-exp over the landmarks folded in order,
// then the fusion weights.  The selection outputs feed the routing and chunk-attention kernels
// of the plain forward.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

template <typename T>
__global__ __launch_bounds__(256) void ml_fixed_selection_kernel(const T* __restrict__ Qs, const T* __restrict__ Klm,
                                                                 const int32_t* __restrict__ idx,
                                                                 float* __restrict__ sel, float* __restrict__ w,
                                                                 int64_t rows, int L, int N, int d, int m, int k,
                                                                 float scale) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int64_t bh = row / L;
  const int k1 = k + 1;
  float mx = -INFINITY;
  for (int r = 0; r < k1; ++r) {
    const int j = idx[row * k1 + r];
    float s = -INFINITY;
    if (j >= 0 && j < N) {
      float amx = -INFINITY, z = 0.f;
      for (int u = 0; u < m; ++u) {
        const T* lp = Klm + ((bh * N + j) * m + u) * d;
        float dot = 0.f;
        for (int e = 0; e < d; ++e) dot += Elem<T>::to_f32(Qs, row * d + e) * Elem<T>::to_f32(lp, e);
        const float a = scale * dot, hi = fmaxf(amx, a), ex = __expf(fminf(amx, a) - hi);
        z = a > amx ? z * ex + 1.f : z + ex;
        amx = hi;
      }
      s = m == 1 ? amx : amx + __logf(z);
    }
    sel[row * k1 + r] = s;
    mx = fmaxf(mx, s);
  }
  float den = 0.f;
  for (int r = 0; r < k1; ++r) den += idx[row * k1 + r] >= 0 ? __expf(sel[row * k1 + r] - mx) : 0.f;
  for (int r = 0; r < k1; ++r)
    if (w) w[row * k1 + r] = idx[row * k1 + r] >= 0 ? __expf(sel[row * k1 + r] - mx) / den : 0.f;
}

hipError_t launch_ml_selection(int dt, int d, const void* Qs, const void* Klm, int m, int32_t* idx, float* sel,
                               float* w, int BH, int L, int N, int k, int select, float scale, hipStream_t st) {
  if (select) return launch_topk_ml(dt, d, Qs, Klm, m, idx, sel, w, BH, L, N, k, scale, st);
  const int64_t rows = (int64_t)BH * L;
  const dim3 grid((unsigned)((rows + 255) / 256));
  if (dt == 0)
    HILS_LAUNCH("ml_fixed_selection", ml_fixed_selection_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)Qs,
                (const bf16_t*)Klm, idx, sel, w, rows, L, N, d, m, k, scale);
  else
    HILS_LAUNCH("ml_fixed_selection", ml_fixed_selection_kernel<float>, grid, dim3(256), 0, st, (const float*)Qs,
                (const float*)Klm, idx, sel, w, rows, L, N, d, m, k, scale);
  return hipGetLastError();
}

}  // namespace hils

namespace hils {

// Backward of the log-sum-exp chunk scores.  For a pair (query t, kept chunk j) with score gradient
// ds (from dq_reduce) and landmark shares p_u = softmax_u(scale qs_t . Klm_j,u):
//   ml_klm_bwd  one workgroup per (chunk, head), the chunk's pairs in routing order (its own queries
//               first): dKlm_j,u = scale * sum ds p_u qs_t.  Four lanes per pair split the head
//               dimension; the chunk's landmark rows sit in LDS.  Deterministic, no atomics.
// The query side, dQs_t += scale * sum over slots of ds sum_u p_u Klm_j,u, is formed by the
// backward's dq_reduce, where ds is made.
template <typename T, int D, int MM>
__global__ __launch_bounds__(256) void ml_klm_bwd_kernel(const T* __restrict__ Qs, const T* __restrict__ Klm,
                                                         const float* __restrict__ ds,
                                                         const int* __restrict__ chunk_off,
                                                         const int* __restrict__ pairs, float* __restrict__ dKlm,
                                                         int L, int N, int k, int m, float scale) {
  constexpr int QD = D / 4;
  constexpr int EPP = 16 / Elem<T>::bytes;
  __shared__ float lmv[MM][D];
  __shared__ float red[64][D + 1];
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int p = tid >> 2, qt = tid & 3;
  const int k1 = k + 1;
  for (int i = tid; i < m * D; i += 256)
    lmv[i / D][i % D] = Elem<T>::to_f32(Klm, ((int64_t)bh * N + j) * m * D + i);
  __syncthreads();
  const int* co = chunk_off + (int64_t)bh * (N + 1);
  const int p_begin = co[j], p_end = co[j + 1];
  const int* pl = pairs + (int64_t)bh * L * k;
  const int ntiles = 1 + (p_end - p_begin + 63) / 64;
  float acc[MM][QD];
#pragma unroll
  for (int u = 0; u < MM; ++u)
#pragma unroll
    for (int e = 0; e < QD; ++e) acc[u][e] = 0.f;
  // TB tiles at a time: their pair entries are requested together, then their ds values and query
  // rows (two memory round trips a batch instead of two a tile); the sums still run tile by tile in
  // list order.  Lanes past the chunk's pairs read a valid row and add nothing.
  constexpr int TB = QD / EPP <= 2 ? 8 : 4;
  const int64_t npl = (int64_t)L * k;
  for (int tb = 0; tb < ntiles; tb += TB) {
    int pe[TB];
#pragma unroll
    for (int v = 0; v < TB; ++v) {
      const int64_t pp = (int64_t)p_begin + (int64_t)(tb + v - 1) * 64 + p;
      pe[v] = pl[pp < 0 ? 0 : (pp < npl ? pp : npl - 1)];
    }
    bool ok[TB];
    float dsb[TB];
    int4 raw[TB][QD / EPP];
#pragma unroll
    for (int v = 0; v < TB; ++v) {
      const int tile = tb + v;
      int t, slot;
      if (tile == 0) {
        t = j * 64 + p;
        slot = k;
        ok[v] = true;
      } else {
        ok[v] = tile < ntiles && p_begin + (tile - 1) * 64 + p < p_end;
        t = ok[v] ? (pe[v] >> 5) : j * 64;
        slot = ok[v] ? (pe[v] & 31) : 0;
      }
      const int64_t row = (int64_t)bh * L + t;
      dsb[v] = ds[row * k1 + slot];
      const T* qp = Qs + row * D + qt * QD;
#pragma unroll
      for (int w = 0; w < QD / EPP; ++w) raw[v][w] = *reinterpret_cast<const int4*>(qp + w * EPP);
    }
#pragma unroll
    for (int v = 0; v < TB; ++v) {
      // all four lanes of a pair take the same branch, so the shuffles below stay within valid pairs
      if (!ok[v]) continue;
      const float dsv = dsb[v];
      float qv[QD];
#pragma unroll
      for (int w = 0; w < QD / EPP; ++w) {
        T vals[EPP];
        __builtin_memcpy(vals, &raw[v][w], 16);
#pragma unroll
        for (int e = 0; e < EPP; ++e) qv[w * EPP + e] = Elem<T>::to_f32(vals, e);
      }
      float a[MM], amax = -INFINITY;
#pragma unroll
      for (int u = 0; u < MM; ++u) {
        float dot = 0.f;
        if (u < m) {
#pragma unroll
          for (int e = 0; e < QD; ++e) dot += qv[e] * lmv[u][qt * QD + e];
        }
        dot += lane_xor(dot, 1);
        dot += lane_xor(dot, 2);
        a[u] = scale * dot;
        if (u < m) amax = fmaxf(amax, a[u]);
      }
      float z = 0.f;
#pragma unroll
      for (int u = 0; u < MM; ++u) z += u < m ? __expf(a[u] - amax) : 0.f;
      const float gsc = dsv / z;
#pragma unroll
      for (int u = 0; u < MM; ++u) {
        const float cu = u < m ? gsc * __expf(a[u] - amax) : 0.f;
#pragma unroll
        for (int e = 0; e < QD; ++e) acc[u][e] += cu * qv[e];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < MM; ++u) {
    if (u >= m) break;  // uniform over the workgroup
    __syncthreads();
#pragma unroll
    for (int e = 0; e < QD; ++e) red[p][qt * QD + e] = acc[u][e];
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
      for (int q = 0; q < 64; ++q) s += red[q][tid];
      dKlm[(((int64_t)bh * N + j) * m + u) * D + tid] = scale * s;
    }
  }
}

template <typename T, int D, int MM>
static hipError_t ml_bwd_mm(const void* Qs, const void* Klm, int m, const float* ds, const int* chunk_off,
                            const int* pairs, float* dKlm, int BH, int L, int N, int k, float scale, hipStream_t st) {
  HILS_LAUNCH("ml_klm_bwd", (ml_klm_bwd_kernel<T, D, MM>), dim3(N, BH), dim3(256), 0, st, (const T*)Qs,
              (const T*)Klm, ds, chunk_off, pairs, dKlm, L, N, k, m, scale);
  return hipGetLastError();
}

// the landmark count rounded up to 2 or 4 sizes the per-lane accumulators
template <typename T, int D>
static hipError_t ml_bwd_t(const void* Qs, const void* Klm, int m, const float* ds, const int* chunk_off,
                           const int* pairs, float* dKlm, int BH, int L, int N, int k, float scale, hipStream_t st) {
  return m <= 2 ? ml_bwd_mm<T, D, 2>(Qs, Klm, m, ds, chunk_off, pairs, dKlm, BH, L, N, k, scale, st)
                : ml_bwd_mm<T, D, 4>(Qs, Klm, m, ds, chunk_off, pairs, dKlm, BH, L, N, k, scale, st);
}

hipError_t launch_ml_bwd(int dt, int d, const void* Qs, const void* Klm, int m, const float* ds, const int* chunk_off,
                         const int* pairs, float* dKlm, int BH, int L, int N, int k, float scale, hipStream_t st) {
  if (m < 1 || m > 4) return hipErrorInvalidValue;
  if (dt == 0)
    return d == 64 ? ml_bwd_t<bf16_t, 64>(Qs, Klm, m, ds, chunk_off, pairs, dKlm, BH, L, N, k, scale, st)
                   : ml_bwd_t<bf16_t, 128>(Qs, Klm, m, ds, chunk_off, pairs, dKlm, BH, L, N, k, scale, st);
  return d == 64 ? ml_bwd_t<float, 64>(Qs, Klm, m, ds, chunk_off, pairs, dKlm, BH, L, N, k, scale, st)
                 : ml_bwd_t<float, 128>(Qs, Klm, m, ds, chunk_off, pairs, dKlm, BH, L, N, k, scale, st);
}

}  // namespace hils
