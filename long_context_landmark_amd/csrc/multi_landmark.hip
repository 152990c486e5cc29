// Several landmarks per chunk: the HiLS summary page (ai-feeds, "Method" > "Input & chunking")
// gives a chunk a few landmarks (usually its first and last token) and "Key modules" item 1 a
// softmax over a chunk's landmark scores before the chunk-level one.  Read as: the chunk score is
// the log-sum-exp of the chunk's m landmark scores.  K_lm is [B][H][N][m][d].
//
//   ml_scores   one workgroup per (64 queries, 64 chunks, head) tile on or below the causal
//               diagonal: for every landmark the 64 x 64 score tile on MFMA (16x16x32 bf16 or
//               16x16x4 fp32; each wave 16 chunks x 64 queries, operands straight from HBM), folded
//               into a running log-sum-exp per (query, chunk) in registers.  Writes the causal chunk
//               scores S [BH][L][N] (fp32).
//   ml_select   one wave per query row: the m = min(k, c) best past chunks by (score desc, index
//               asc) in k rounds of a group maximum over 64-bit keys (16 lanes per row when the
//               row has at most 128 chunks and k < 16, else a wave; keys held in registers up to
//               512 chunks), the own chunk's score, and
//               the fusion weights; or, for a caller-given selection, its scores and weights.
// The selection outputs then feed the routing and chunk-attention kernels of the plain forward.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

template <typename T, int D>
__global__ __launch_bounds__(256) void ml_scores_kernel(const T* __restrict__ Qs, const T* __restrict__ Klm,
                                                        float* __restrict__ S, int L, int N, int m, float scale) {
  const int bh = blockIdx.z;
  const int t0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  if (j0 > t0 / 64) return;  // no causal chunk in this tile
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const T* Qb = Qs + (int64_t)bh * L * D;
  const int jrow = j0 + 16 * w + r16;
  float mx[4][4], z[4][4];
  for (int u = 0; u < m; ++u) {
    f32x4_t acc[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) acc[qb] = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      Frag<T> a;
      if (jrow < N) a.load(Klm + (((int64_t)bh * N + jrow) * m + u) * D + ks * 32 + 8 * g);
      else a.zero();
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        Frag<T> b;
        b.load(Qb + (int64_t)(t0 + 16 * qb + r16) * D + ks * 32 + 8 * g);
        mma(acc[qb], a, b);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = scale * acc[qb][i];
        if (u == 0) {
          mx[qb][i] = a;
          z[qb][i] = 1.f;
        } else if (a > mx[qb][i]) {
          z[qb][i] = z[qb][i] * __expf(mx[qb][i] - a) + 1.f;
          mx[qb][i] = a;
        } else {
          z[qb][i] += __expf(a - mx[qb][i]);
        }
      }
  }
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int t = t0 + 16 * qb + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 16 * w + 4 * g + i;
      if (j < N && j <= t / 64) S[((int64_t)bh * L + t) * N + j] = m == 1 ? mx[qb][i] : mx[qb][i] + __logf(z[qb][i]);
    }
  }
}

// G lanes per query row (64 / G rows per wave).  VPL > 0: every candidate of a row fits in VPL keys per
// lane (c <= G VPL), loaded once; VPL = 0: the row is re-read from memory in every round.  Lane gl of a
// row's group ends up holding slot gl (gl < k) and, if gl == k, the own chunk; G > k is required.
template <int VPL, int G>
__global__ __launch_bounds__(256) void ml_select_kernel(const float* __restrict__ S, int32_t* __restrict__ idx,
                                                        float* __restrict__ sel, float* __restrict__ w, int64_t rows,
                                                        int L, int N, int k, int select) {
  const int lane = threadIdx.x & 63, gl = lane % G;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  // rows past the end compute alongside (every lane takes part in the group shuffles) and write nothing
  const bool live = row < rows;
  const int64_t rr = live ? row : rows - 1;
  const int t = (int)(rr % L);
  const int c = t / 64;
  const int m = min(k, c);
  const int k1 = k + 1;
  const float* srow = S + rr * N;
  const int64_t base = rr * k1;
  int ix = -1;
  float sv = -INFINITY;
  if (select) {
    uint64_t keys[VPL > 0 ? VPL : 1];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int j = gl + G * i;
      keys[i] = j < c ? make_key(srow[j], j) : 0ull;
    }
    uint64_t prev = ~0ull;
    // m differs between the rows of a wave: every group runs k rounds, extra ones find nothing new
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0ull;
      if (VPL > 0) {
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (keys[i] < prev && keys[i] > best) best = keys[i];
      } else {
        for (int j = gl; j < c; j += G) {
          const uint64_t key = make_key(srow[j], j);
          if (key < prev && key > best) best = key;
        }
      }
#pragma unroll
      for (int msk = 1; msk < G; msk <<= 1) {
        const uint64_t o = shfl_xor_u64(best, msk);
        best = o > best ? o : best;
      }
      if (gl == r && r < m) {
        ix = key_index(best);
        sv = key_score(best);
      }
      prev = best;
    }
  } else if (gl < k) {
    ix = idx[base + gl];
    if (ix >= 0) sv = srow[ix];
  }
  if (gl == k) {
    ix = c;
    sv = srow[c];
  }
  const bool used = gl <= k && ix >= 0;
  float smax = used ? sv : -INFINITY;
#pragma unroll
  for (int msk = 1; msk < G; msk <<= 1) smax = fmaxf(smax, lane_xor(smax, msk));
  const float ev = used ? __expf(sv - smax) : 0.f;
  float den = ev;
#pragma unroll
  for (int msk = 1; msk < G; msk <<= 1) den += lane_xor(den, msk);
  if (live && gl <= k) {
    if (select) idx[base + gl] = ix;
    sel[base + gl] = used ? sv : -INFINITY;
    if (w) w[base + gl] = ev / den;
  }
}

template <typename T, int D>
static hipError_t ml_scores_t(const void* Qs, const void* Klm, float* S, int BH, int L, int N, int m, float scale,
                              hipStream_t st) {
  HILS_LAUNCH("ml_scores", (ml_scores_kernel<T, D>), dim3(L / 64, (N + 63) / 64, BH), dim3(256), 0, st,
              (const T*)Qs, (const T*)Klm, S, L, N, m, scale);
  return hipGetLastError();
}

hipError_t launch_ml_selection(int dt, int d, const void* Qs, const void* Klm, int m, float* S, int32_t* idx,
                               float* sel, float* w, int BH, int L, int N, int k, int select, float scale,
                               hipStream_t st) {
  // with at most two landmark tiles per query chunk the selection kernel forms the log-sum-exp
  // scores itself and no score matrix is written
  if (select && topk_ml_fused(N)) return launch_topk_ml(dt, d, Qs, Klm, m, idx, sel, w, BH, L, N, k, scale, st);
  hipError_t e;
  if (dt == 0)
    e = d == 64 ? ml_scores_t<bf16_t, 64>(Qs, Klm, S, BH, L, N, m, scale, st)
                : ml_scores_t<bf16_t, 128>(Qs, Klm, S, BH, L, N, m, scale, st);
  else
    e = d == 64 ? ml_scores_t<float, 64>(Qs, Klm, S, BH, L, N, m, scale, st)
                : ml_scores_t<float, 128>(Qs, Klm, S, BH, L, N, m, scale, st);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)BH * L;
  if (N <= 128 && k < 16) {
    // 16 lanes per row, eight keys each: four rows share a wave and its shuffles
    const dim3 grid((unsigned)((rows + 15) / 16));
    HILS_LAUNCH("ml_select", (ml_select_kernel<8, 16>), grid, dim3(256), 0, st, S, idx, sel, w, rows, L, N, k,
                select);
  } else {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (N <= 512)
      HILS_LAUNCH("ml_select", (ml_select_kernel<8, 64>), grid, dim3(256), 0, st, S, idx, sel, w, rows, L, N, k,
                  select);
    else
      HILS_LAUNCH("ml_select", (ml_select_kernel<0, 64>), grid, dim3(256), 0, st, S, idx, sel, w, rows, L, N, k,
                  select);
  }
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
