// Landmark scoring and causal top-k chunk selection (HiLS attention, step 1-2).
//
// Passages defining the operation:
//   "Hierarchical Sparse Attention Done Right" (ai-feeds summary), section
//   "Method" > "Key modules" item 1 (each query scores the chunks through
//   their landmark representation; chunk-level softmax gives the retrieval
//   weights) and item 2 (the query keeps the top-k chunks);
//   paper.oopus.info review, section 2 (one landmark token per chunk scored by
//   the current query; the highest scoring chunks are read in detail).
// Fixed here: score = scale * <q_t, Klm_j> with scale = 1/sqrt(d) by default;
// candidates of query t are the completed past chunks j < t/64; ties go to
// the lower chunk index; the own chunk t/64 is always added, scored by its
// own landmark, and not counted in k.
//
// Scores are a dense contraction Q . Klm^T, so they run on bf16 MFMA with
// fp32 accumulation.  Selection never materialises the score matrix: a first
// sweep keeps, per query, the running maximum of each of 64 residue groups
// (chunk index mod 64).  The m-th largest of those maxima is a lower bound on
// the m-th largest score (the maxima are m distinct candidates), so a second
// sweep, which recomputes bit-identical scores, only has to keep candidates at
// or above it.  The exact top-m is then sorted out of the few survivors.  A
// query with more survivors than fit in LDS (possible only with many exactly
// tied scores) falls back to m exact arg-max sweeps.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

// ----------------------------------------------------------------------------
// Dense causal scores S[b,h,t,j] (fp32; -inf for j > t/64).  One workgroup per
// 64 queries x 64 chunks; wave w takes the 16-chunk block w of the tile and all
// 64 queries (4 column blocks), matching the selection kernel's arithmetic.
template <typename T, int D>
__global__ __launch_bounds__(256) void landmark_scores_kernel(const T* __restrict__ Q, const T* __restrict__ Klm,
                                                              float* __restrict__ S, int L, int N, float scale) {
  const int bh = blockIdx.z;
  const int t0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const T* Qb = Q + (int64_t)bh * L * D;
  const T* Kb = Klm + (int64_t)bh * N * D;
  const int jrow = j0 + 16 * w + r16;
  f32x4_t acc[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) acc[qb] = zero4();
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    Frag<T> a;
    if (jrow < N) a.load(Kb + (int64_t)jrow * D + ks * 32 + 8 * g);
    else a.zero();
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int tq = t0 + 16 * qb + r16;
      Frag<T> b;
      if (tq < L) b.load(Qb + (int64_t)tq * D + ks * 32 + 8 * g);
      else b.zero();
      mma(acc[qb], a, b);
    }
  }
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int t = t0 + 16 * qb + r16;
    if (t >= L) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 16 * w + 4 * g + i;
      if (j < N) S[((int64_t)bh * L + t) * N + j] = (j <= t / 64) ? scale * acc[qb][i] : -INFINITY;
    }
  }
}

constexpr int TK_CAP = 64;  // survivor slots per query (16 per sorting lane)

// One workgroup per (b,h, query chunk c): the 64 queries t = 64c .. 64c+63
// share the candidate set {0..c-1}.  Wave w scores the 16-chunk block w of
// every 64-chunk landmark tile against all 64 queries.
// SMALL: every query chunk has at most two landmark tiles of candidates (N <= 129 chunks);
// the score tiles of sweep 1 are then kept in registers for sweep 2.
template <typename T, int D, bool SMALL>
__global__ __launch_bounds__(256, (SMALL && D == 64) ? 4 : 3) void topk_select_kernel(const T* __restrict__ Q, const T* __restrict__ Klm,
                                                          int32_t* __restrict__ idx, float* __restrict__ sel,
                                                          float* __restrict__ wout, int L, int N, int k,
                                                          float scale) {
  const int nc = L / 64;
  int xi, bh;
  xcd_map(xi, bh);  // a head's landmark rows are re-read by all its query chunks: keep them in one L2
  const int c = nc - 1 - xi;  // longest candidate lists first
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const int m = min(k, c);
  const int k1 = k + 1;
  const T* Qb = Q + ((int64_t)bh * L + (int64_t)c * 64) * D;
  const T* Kb = Klm + (int64_t)bh * N * D;

  // the group maxima (sweep 1), the survivors (sweep 2) and the sorted top keys share storage
  __shared__ union {
    float gmax[64][65];
    uint64_t surv[64][TK_CAP];
    uint64_t top[64][16];
  } u_s;
  auto& gmax_s = u_s.gmax;
  auto& surv = u_s.surv;
  auto& top_s = u_s.top;
  __shared__ int cnt_s[64];
  __shared__ float tau_s[64];
  __shared__ int ovf_s;

  Frag<T> qf[4][D / 32];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[qb][ks].load(Qb + (int64_t)(16 * qb + r16) * D + ks * 32 + 8 * g);

  const int ntile = (c + 63) / 64;
  // scores of chunks tile*64 + 16w + 4g + i (i = 0..3) for queries 16qb + r16; the landmark
  // fragments of the next tile are loaded while the current one is on the MFMA units
  // rows past the candidates (j >= c) load row c-1 instead: their scores are never used, and
  // unconditional loads let the compiler wait for exactly the tile it needs
  auto load_tile = [&](int tile, Frag<T>(&a)[D / 32]) {
    const int jrow = min(tile * 64 + 16 * w + r16, c - 1);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) a[ks].load(Kb + (int64_t)jrow * D + ks * 32 + 8 * g);
  };
  // the four query blocks' products are independent: issuing them in turn keeps the
  // MFMA pipeline full instead of waiting on each accumulator
  auto mma_tile = [&](const Frag<T>(&a)[D / 32], f32x4_t(&acc)[4]) {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) acc[qb] = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) mma(acc[qb], a[ks], qf[qb][ks]);
  };
  // the next tile is always requested (the last one again at the end) so that every wait
  // covers exactly the tile about to be used; the scheduling barriers keep those requests
  // ahead of the current tile's products, a whole tile of work before they are needed
  auto sweep_from = [&](Frag<T>(&a0)[D / 32], auto&& visit) {
    Frag<T> a1[D / 32];
    for (int i = 0; i < ntile; i += 2) {
      f32x4_t acc[4];
      load_tile(min(i + 1, ntile - 1), a1);
      __builtin_amdgcn_sched_barrier(0);
      mma_tile(a0, acc);
      visit(i, acc);
      load_tile(min(i + 2, ntile - 1), a0);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < ntile) {
        mma_tile(a1, acc);
        visit(i + 1, acc);
      }
    }
  };
  auto sweep = [&](auto&& visit) {
    Frag<T> a0[D / 32];
    load_tile(0, a0);
    sweep_from(a0, visit);
  };

  // the first landmark tile and the own-chunk operands are requested before anything waits
  Frag<T> first_tile[D / 32], second_tile[SMALL ? D / 32 : 1];
  if (m > 0) {
    load_tile(0, first_tile);
    if constexpr (SMALL) load_tile(min(1, ntile - 1), second_tile);
  }
  __shared__ float own_s[64];
  {
    const int q = tid >> 2, part = tid & 3;
    Frag<T> oq[D / 32], ol[D / 32];
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      oq[u].load(Qb + (int64_t)q * D + part * (D / 4) + 8 * u);
      ol[u].load(Kb + (int64_t)c * D + part * (D / 4) + 8 * u);
    }
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += oq[u].get(e) * ol[u].get(e);
    dot += lane_xor(dot, 1);
    dot += lane_xor(dot, 2);
    if (part == 0) own_s[q] = scale * dot;
  }

  if (tid == 0) ovf_s = 0;
  if (tid < 64) cnt_s[tid] = 0;

  if (m > 0) {
    // With at most two landmark tiles (c <= 128) both score tiles stay in registers and the
    // second sweep reads them there; longer candidate lists recompute them.
    f32x4_t keep0[SMALL ? 4 : 1], keep1[SMALL ? 4 : 1];
    // sweep 1: per-group running maxima of the raw accumulators (the scale is positive, so
    // the maximum commutes with the monotonic rounded multiplication applied once below)
    float gm[4][4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) gm[qb][i] = -INFINITY;
    auto group_max = [&](int tile, const f32x4_t(&acc)[4]) {
      if ((tile + 1) * 64 <= c) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) gm[qb][i] = fmaxf(gm[qb][i], acc[qb][i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = tile * 64 + 16 * w + 4 * g + i;
          if (j < c) {
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) gm[qb][i] = fmaxf(gm[qb][i], acc[qb][i]);
          }
        }
      }
    };
    if constexpr (SMALL) {
      mma_tile(first_tile, keep0);
      mma_tile(second_tile, keep1);
      group_max(0, keep0);
      if (ntile > 1) group_max(1, keep1);
    } else {
      sweep_from(first_tile, [&](int tile, f32x4_t(&acc)[4]) { group_max(tile, acc); });
    }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) gmax_s[16 * qb + r16][16 * w + 4 * g + i] = scale * gm[qb][i];
    __syncthreads();
    {
      const int q = tid >> 2, part = tid & 3;
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = gmax_s[q][16 * part + e];
      sort16_desc(v);
      merge16_with_lane(v, 1);
      merge16_with_lane(v, 2);
      float tau = v[0];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (e == m - 1) tau = v[e];
      if (part == 0) tau_s[q] = tau;
    }
    __syncthreads();
    // sweep 2: keep candidates at or above the bound.  A raw-accumulator bound a little below
    // tau / scale first rejects whole rows of four (every score that reaches tau after the
    // rounded scaling passes it: the margin exceeds the rounding of both quotients); the few
    // that pass are then tested exactly on the scaled score.
    float tau_r[4], raw_lo[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      tau_r[qb] = tau_s[16 * qb + r16];
      const float t = tau_r[qb] / scale;
      raw_lo[qb] = t - fabsf(t) * 1e-6f - 1e-30f;
    }
    __syncthreads();  // every lane has read its bounds: the survivor buffer may overwrite the maxima
    auto survive = [&](int tile, const f32x4_t(&acc)[4]) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const float m4 = fmaxf(fmaxf(acc[qb][0], acc[qb][1]), fmaxf(acc[qb][2], acc[qb][3]));
        if (m4 >= raw_lo[qb]) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = tile * 64 + 16 * w + 4 * g + i;
            const float sv = scale * acc[qb][i];
            if (j < c && sv >= tau_r[qb]) {
              const int q = 16 * qb + r16;
              const int p = atomicAdd(&cnt_s[q], 1);
              if (p < TK_CAP) surv[q][p] = make_key(sv, j);
            }
          }
        }
      }
    };
    if constexpr (SMALL) {
      survive(0, keep0);
      if (ntile > 1) survive(1, keep1);
    } else {
      sweep([&](int tile, f32x4_t(&acc)[4]) { survive(tile, acc); });
    }
    __syncthreads();
    // exact top-m among the survivors: 4 lanes per query, 16 slots each.  When every query
    // of the wavefront has at most 16 (or 32) survivors, one (two) of its lanes hold them all
    // and the merges between lanes that hold nothing are skipped.
    {
      const int q = tid >> 2, part = tid & 3;
      const int n = cnt_s[q];
      int nmax = n;
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) nmax = max(nmax, lane_xor(nmax, msk));
      uint64_t v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int p = 16 * part + e;
        v[e] = (p < n && p < TK_CAP) ? surv[q][p] : 0ull;
      }
      sort16_desc(v);
      if (nmax > 16) merge16_with_lane(v, 1);
      if (nmax > 32) merge16_with_lane(v, 2);
      __syncthreads();  // every survivor has been read: the sorted keys overwrite the buffer
      if (part == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) top_s[q][e] = v[e];
        if (n > TK_CAP) atomicOr(&ovf_s, 1);
      }
    }
    __syncthreads();
    if (ovf_s) {
      // exact fallback: for each rank, the largest key below the previous one
      __shared__ uint64_t best_s[64];
      __shared__ uint64_t prev_s[64];
      __shared__ int redo_s[64];
      if (tid < 64) {
        redo_s[tid] = cnt_s[tid] > TK_CAP;
        prev_s[tid] = ~0ull;
      }
      __syncthreads();
      for (int r = 0; r < m; ++r) {
        if (tid < 64) best_s[tid] = 0ull;
        __syncthreads();
        sweep([&](int tile, f32x4_t(&acc)[4]) {
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) {
            const int q = 16 * qb + r16;
            if (!redo_s[q]) continue;
            const uint64_t prev = prev_s[q];
            uint64_t best = 0ull;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = tile * 64 + 16 * w + 4 * g + i;
              if (j < c) {
                const uint64_t key = make_key(scale * acc[qb][i], j);
                if (key < prev && key > best) best = key;
              }
            }
            if (best) atomicMax((unsigned long long*)&best_s[q], (unsigned long long)best);
          }
        });
        __syncthreads();
        if (tid < 64 && redo_s[tid]) {
          top_s[tid][r] = best_s[tid];
          prev_s[tid] = best_s[tid];
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();

  // fusion weights and outputs: the softmax statistics per query, then the 64 query rows of
  // each output, which are consecutive in memory, written element by element across the
  // workgroup (coalesced)
  __shared__ float mx_s[64], inv_s[64];
  if (tid < 64) {
    const int q = tid;
    const float s_own = own_s[q];
    float mx = s_own;
    for (int r = 0; r < m; ++r) mx = fmaxf(mx, key_score(top_s[q][r]));
    float den = __expf(s_own - mx);
    for (int r = 0; r < m; ++r) den += __expf(key_score(top_s[q][r]) - mx);
    mx_s[q] = mx;
    inv_s[q] = 1.f / den;
  }
  __syncthreads();
  const int64_t base = ((int64_t)bh * L + (int64_t)c * 64) * k1;
  for (int e = tid; e < 64 * k1; e += 256) {
    const int q = e / k1, r = e % k1;
    int ix;
    float sv, wv;
    if (r == k) {
      ix = c;
      sv = own_s[q];
      wv = __expf(sv - mx_s[q]) * inv_s[q];
    } else if (r < m) {
      const uint64_t key = top_s[q][r];
      ix = key_index(key);
      sv = key_score(key);
      wv = __expf(sv - mx_s[q]) * inv_s[q];
    } else {
      ix = -1;
      sv = -INFINITY;
      wv = 0.f;
    }
    idx[base + e] = ix;
    sel[base + e] = sv;
    if (wout) wout[base + e] = wv;
  }
}

template <typename T, int D>
hipError_t launch_landmark_scores_t(const void* Q, const void* Klm, float* S, int BH, int L, int N, float scale,
                                    hipStream_t st) {
  dim3 grid((L + 63) / 64, (N + 63) / 64, BH);
  HILS_LAUNCH("landmark_scores", (landmark_scores_kernel<T, D>), grid, dim3(256), 0, st, (const T*)Q, (const T*)Klm, S, L, N,
                     scale);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_topk_t(const void* Q, const void* Klm, int32_t* idx, float* sel, float* w, int BH, int L, int N,
                         int k, float scale, hipStream_t st) {
  dim3 grid(L / 64, BH);
  if (N <= 129)
    HILS_LAUNCH("topk_select", (topk_select_kernel<T, D, true>), grid, dim3(256), 0, st, (const T*)Q, (const T*)Klm, idx,
                sel, w, L, N, k, scale);
  else
    HILS_LAUNCH("topk_select", (topk_select_kernel<T, D, false>), grid, dim3(256), 0, st, (const T*)Q, (const T*)Klm, idx,
                sel, w, L, N, k, scale);
  return hipGetLastError();
}

hipError_t launch_landmark_scores(int dt, int d, const void* Q, const void* Klm, float* S, int BH, int L, int N,
                                  float scale, hipStream_t st) {
  if (dt == 0) return d == 64 ? launch_landmark_scores_t<bf16_t, 64>(Q, Klm, S, BH, L, N, scale, st)
                              : launch_landmark_scores_t<bf16_t, 128>(Q, Klm, S, BH, L, N, scale, st);
  return d == 64 ? launch_landmark_scores_t<float, 64>(Q, Klm, S, BH, L, N, scale, st)
                 : launch_landmark_scores_t<float, 128>(Q, Klm, S, BH, L, N, scale, st);
}

hipError_t launch_topk(int dt, int d, const void* Q, const void* Klm, int32_t* idx, float* sel, float* w, int BH,
                       int L, int N, int k, float scale, hipStream_t st) {
  if (dt == 0) return d == 64 ? launch_topk_t<bf16_t, 64>(Q, Klm, idx, sel, w, BH, L, N, k, scale, st)
                              : launch_topk_t<bf16_t, 128>(Q, Klm, idx, sel, w, BH, L, N, k, scale, st);
  return d == 64 ? launch_topk_t<float, 64>(Q, Klm, idx, sel, w, BH, L, N, k, scale, st)
                 : launch_topk_t<float, 128>(Q, Klm, idx, sel, w, BH, L, N, k, scale, st);
}

}  // namespace hils
