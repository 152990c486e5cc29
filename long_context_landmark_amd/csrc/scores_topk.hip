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
// or above it.  The exact top-m is then ranked out of the few survivors.  A
// query with more survivors than fit in LDS (possible only with many exactly
// tied scores) falls back to m exact arg-max sweeps.
// With several landmarks per chunk (the summary's "Input & chunking" and "Key
// modules" item 1) a chunk's score is the log-sum-exp of its landmark scores;
// the selection kernel forms those itself from the MFMA products of every
// landmark (topk_select_ml), in both sweeps, so no score matrix is written.
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

// ----------------------------------------------------------------------------
// Landmark rows in MFMA fragment order (bf16).  The selection sweeps read every landmark
// tile once per 64-query block; loaded straight from [N][D] rows, a fragment load has each
// lane quad spread over four rows, which the vector memory path serves at a quarter of its
// rate.  This copy stores, for every 16-row block and 32-element k-step, the 64 lanes'
// 16-byte pieces one after another (lane = r16 + 16 g holds row r16, elements 8g..8g+7 of
// the step), so one fragment load reads 1 KiB of consecutive bytes.  Rows are padded to a
// multiple of 64 with zeros.  Layout: [BH][Npad / 16][D / 32][64][8].
__host__ __device__ inline int klm_frag_rows(int N) { return (N + 63) / 64 * 64; }

template <int D>
__global__ __launch_bounds__(256) void klm_frag_kernel(const bf16_t* __restrict__ Klm, bf16_t* __restrict__ F, int N,
                                                       int Npad, int64_t total_pieces) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= total_pieces) return;
  constexpr int KS = D / 32;
  const int lane = (int)(p & 63);
  const int ks = (int)((p >> 6) % KS);
  const int64_t blk_all = (p >> 6) / KS;  // bh * (Npad / 16) + block
  const int nblk = Npad / 16;
  const int64_t bh = blk_all / nblk;
  const int row = (int)(blk_all % nblk) * 16 + (lane & 15);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row < N) v = *reinterpret_cast<const u32x4_t*>(Klm + (bh * N + row) * D + ks * 32 + 8 * (lane >> 4));
  *reinterpret_cast<u32x4_t*>(F + p * 8) = v;
}

// Neighbouring floats in the order of the reals (-0 and +0 are adjacent steps).
__device__ __forceinline__ float float_step(float x, int dir) {
  const int i = __float_as_int(x);
  int o = i >= 0 ? i : -(i & 0x7fffffff) - 1;
  o += dir;
  return __int_as_float(o >= 0 ? o : (int)((uint32_t)(-(o + 1)) | 0x80000000u));
}
// The least float a with fl(s * a) >= t, for s > 0: the rounded product is non-decreasing
// in a, so fl(s * x) >= t exactly when x >= a.  Starts at t / s and steps to the boundary
// (a few ulps at most).  Infinite t is returned as it is (the same test then holds).
__device__ __forceinline__ float least_raw_bound(float t, float s) {
  if (!(fabsf(t) < INFINITY)) return t;
  float a = t / s;
  if (s * a >= t) {
    for (int it = 0; it < 64; ++it) {
      const float b = float_step(a, -1);
      if (!(s * b >= t)) break;
      a = b;
    }
  } else {
    for (int it = 0; it < 64 && !(s * a >= t); ++it) a = float_step(a, 1);
  }
  return a;
}

constexpr int TK_CAP = 64;  // survivor slots per query (16 per ranking lane)
constexpr int TK_SMALL_N = 129;  // up to this many chunks a query chunk has at most two candidate tiles

// One workgroup per (b,h, query chunk c): the 64 queries t = 64c .. 64c+63
// share the candidate set {0..c-1}.  Wave w scores the 16-chunk block w of
// every 64-chunk landmark tile against all 64 queries.
// SMALL: every query chunk has at most two landmark tiles of candidates (N <= 129 chunks);
// the score tiles of sweep 1 are then kept in registers for sweep 2.
// ML: mlm landmarks per chunk (rows j * mlm + u); a chunk's score is the log-sum-exp of its landmark
// scores, folded over the landmarks in order, so that the score tiles the sweeps see hold finished
// scores instead of raw products (short lists keep them in registers, long ones recompute them in
// each sweep; long lists read the landmark rows directly, without the fragment-order copy).
template <typename T, int D, bool SMALL, bool ML = false>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? ((SMALL && D == 64) ? 4 : ((ML && D == 128) ? 2 : 3)) : 1) void topk_select_kernel(const T* __restrict__ Q, const T* __restrict__ Klm,
                                                          const T* __restrict__ F, int32_t* __restrict__ idx,
                                                          float* __restrict__ sel, float* __restrict__ wout, int L,
                                                          int N, int k, float scale, int mlm) {
  const int nc = L / 64;
  int xi, bh;
  xcd_map(xi, bh);  // a head's landmark rows are re-read by all its query chunks: keep them in one L2
  const int c = nc - 1 - xi;  // longest candidate lists first
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const int m = min(k, c);
  const int k1 = k + 1;
  const T* Qb = Q + ((int64_t)bh * L + (int64_t)c * 64) * D;
  const int lpc = ML ? mlm : 1;  // landmark rows per chunk
  const T* Kb = Klm + (int64_t)bh * N * lpc * D;
  // the score of a kept value: raw products are scaled here, several-landmark tiles hold scores
  auto sc = [&](float x) { return ML ? x : scale * x; };
  // bf16 landmarks of long candidate lists are read from their fragment-order copy (one
  // 1 KiB run per fragment load); with at most two tiles the direct loads are kept
  constexpr bool FRAG = sizeof(T) == 2 && !SMALL && !ML;
  const T* Fb = FRAG ? F + (int64_t)bh * klm_frag_rows(N) * D : nullptr;

  // the group maxima (sweep 1), the survivors (sweep 2) and the sorted top keys share storage
  __shared__ union {
    float gmax[64][65];
    uint64_t surv[64][TK_CAP + 1];  // rows padded by one key: the lanes of a wave read different
    uint64_t top[64][17];           // queries' rows, which would otherwise share LDS banks
  } u_s;
  auto& gmax_s = u_s.gmax;
  auto& surv = u_s.surv;
  auto& top_s = u_s.top;
  __shared__ int cnt_s[64];
  __shared__ float tau_s[64];
  __shared__ f32x4_t park_s[SMALL ? 1 : 4][4][64];  // survivor sweep: a wave's accumulators
  __shared__ int ovf_s;

  Frag<T> qf[4][D / 32];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[qb][ks].load(Qb + (int64_t)(16 * qb + r16) * D + ks * 32 + 8 * g);

  const int ntile = (c + 63) / 64;
  // scores of chunks tile*64 + 16w + 4g + i (i = 0..3) for queries 16qb + r16; the landmark
  // fragments of the next tile are loaded while the current one is on the MFMA units
  // rows past chunk c load row c instead (row c itself gives the own-chunk score, the others
  // are never used), and unconditional loads let the compiler wait for exactly the tile it needs
  // In the fragment-order copy every tile below ceil(c/64) is whole; its rows at or past c
  // (later chunks, or zero padding) are scored but never used.
  auto load_tile = [&](int tile, Frag<T>(&a)[D / 32], int u = 0) {
    if constexpr (FRAG) {
      const T* fp = Fb + ((int64_t)(4 * tile + w) * (D / 32) * 64 + lane) * 8;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) a[ks].load(fp + ks * 64 * 8);
    } else {
      const int64_t lrow = (int64_t)min(tile * 64 + 16 * w + r16, c) * lpc + u;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) a[ks].load(Kb + lrow * D + ks * 32 + 8 * g);
    }
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
  // Workgroups of neighbouring query chunks run together on one XCD; each starts its sweep
  // at another landmark tile (and wraps around), so that they do not all request the same
  // few L2 lines at once.  The visits are order-independent (maxima, survivor sets).
  const int t_start = SMALL ? 0 : c % max(ntile, 1);
  auto tile_at = [&](int i) { return i + t_start < ntile ? i + t_start : i + t_start - ntile; };
  auto sweep_from = [&](Frag<T>(&a0)[D / 32], auto&& visit) {
    Frag<T> a1[D / 32];
    for (int i = 0; i < ntile; i += 2) {
      f32x4_t acc[4];
      load_tile(tile_at(min(i + 1, ntile - 1)), a1);
      __builtin_amdgcn_sched_barrier(0);
      mma_tile(a0, acc);
      visit(tile_at(i), acc);
      load_tile(tile_at(min(i + 2, ntile - 1)), a0);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < ntile) {
        mma_tile(a1, acc);
        visit(tile_at(i + 1), acc);
      }
    }
  };
  auto sweep = [&](auto&& visit) {
    Frag<T> a0[D / 32];
    load_tile(tile_at(0), a0);
    sweep_from(a0, visit);
  };

  // one landmark's score a folded into the running maximum mx and sum z = sum exp(score - mx)
  // (from mx = -inf, z = 0): one exponential of the lesser minus the greater of a and mx
  auto lse_fold = [](float a, float& mx, float& z) {
    const float hi = fmaxf(mx, a), e = __expf(fminf(mx, a) - hi);
    z = a > mx ? z * e + 1.f : z + e;
    mx = hi;
  };
  // landmark u's score: the first one starts the fold without an exponential (the same values)
  auto lse_fold_u = [&](int u, float a, float& mx, float& z) {
    if (u == 0) {
      mx = a;
      z = 1.f;
    } else {
      lse_fold(a, mx, z);
    }
  };
  // several landmarks, long candidate lists: every tile's landmarks in turn, folded into a running
  // log-sum-exp per (query, chunk) whose result the visitor sees; the next landmark rows (or the
  // next tile's first) are requested before the current products
  auto ml_sweep = [&](auto&& visit) {
    Frag<T> cur[D / 32], nxt[D / 32];
    load_tile(tile_at(0), cur, 0);
    for (int i = 0; i < ntile; ++i) {
      const int tile = tile_at(i);
      float mx[4][4], z[4][4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mx[qb][e] = -INFINITY;
          z[qb][e] = 0.f;
        }
      for (int u = 0; u < mlm; ++u) {
        const bool more = u + 1 < mlm || i + 1 < ntile;
        if (u + 1 < mlm) load_tile(tile, nxt, u + 1);
        else if (i + 1 < ntile) load_tile(tile_at(i + 1), nxt, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          f32x4_t cc = zero4();
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) mma(cc, cur[ks], qf[qb][ks]);
#pragma unroll
          for (int e = 0; e < 4; ++e) lse_fold_u(u, scale * cc[e], mx[qb][e], z[qb][e]);
        }
        if (more) {
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) cur[ks] = nxt[ks];
        }
      }
      f32x4_t acc[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[qb][e] = mlm == 1 ? mx[qb][e] : mx[qb][e] + __logf(z[qb][e]);
      visit(tile, acc);
    }
  };
  // the first landmark tile and the own-chunk operands are requested before anything waits
  Frag<T> first_tile[D / 32], second_tile[SMALL && !ML ? D / 32 : 1];
  if ((SMALL || !ML) && m > 0) {
    load_tile(tile_at(0), first_tile);
    if constexpr (SMALL && !ML) load_tile(min(1, ntile - 1), second_tile);
  }
  // own-chunk scores.  When chunk c lies in the last candidate tile (c not a multiple of 64) the
  // first sweep's products hold them: the lane that holds (query, c) stores them.  Otherwise
  // wave 0 forms them from the query fragments already held: lane (r16, g) takes the elements
  // 8g.. of every 32-element step of query 16 qb + r16, the four lane groups then add their
  // partial products.
  __shared__ float own_s[64];
  const bool own_in_tile = (c & 63) != 0;
  if (ML && !own_in_tile && w == 0) {
    // several landmarks: wave 0 forms the own chunk's landmark scores on the MFMA units, from a
    // tile whose rows all clamp to chunk c, and folds element 0 of each query block
    float omx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, oz[4] = {0.f, 0.f, 0.f, 0.f};
    for (int u = 0; u < mlm; ++u) {
      Frag<T> lf[D / 32];
      load_tile(c / 64, lf, u);
      f32x4_t cc[4];
      mma_tile(lf, cc);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) lse_fold_u(u, scale * cc[qb][0], omx[qb], oz[qb]);
    }
    if (g == 0) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) own_s[16 * qb + r16] = mlm == 1 ? omx[qb] : omx[qb] + __logf(oz[qb]);
    }
  } else if (!ML && !own_in_tile && w == 0) {
    Frag<T> lf[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) lf[ks].load(Kb + (int64_t)c * D + ks * 32 + 8 * g);
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float dot = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += qf[qb][ks].get(e) * lf[ks].get(e);
      dot += lane_xor(dot, 16);
      dot += lane_xor(dot, 32);
      if (g == 0) own_s[16 * qb + r16] = scale * dot;
    }
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
          } else if (j == c) {  // the last, partial tile holds the own chunk
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) own_s[16 * qb + r16] = sc(acc[qb][i]);
          }
        }
      }
    };
    if constexpr (ML && SMALL) {
      // a tile's landmarks in order, folded into a running log-sum-exp that ends in its kept
      // tile; the next landmark rows (or the next tile's first) are requested before the
      // current products.  The second tile runs only when it holds candidates.
      Frag<T> nxt[D / 32];
      auto ml_tile = [&](int tl, f32x4_t(&keep)[4], bool more) {
        float mx[4][4], z[4][4];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            mx[qb][i] = -INFINITY;
            z[qb][i] = 0.f;
          }
        for (int u = 0; u < mlm; ++u) {
          const bool next = u + 1 < mlm || more;
          if (u + 1 < mlm) load_tile(tl, nxt, u + 1);
          else if (more) load_tile(tl + 1, nxt, 0);
          __builtin_amdgcn_sched_barrier(0);
          // one query block at a time: its products are folded before the next block's are formed
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) {
            f32x4_t cc = zero4();
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) mma(cc, first_tile[ks], qf[qb][ks]);
#pragma unroll
            for (int i = 0; i < 4; ++i) lse_fold(scale * cc[i], mx[qb][i], z[qb][i]);
          }
          if (next) {
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) first_tile[ks] = nxt[ks];
          }
        }
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) keep[qb][i] = mlm == 1 ? mx[qb][i] : mx[qb][i] + __logf(z[qb][i]);
      };
      ml_tile(0, keep0, ntile > 1);
      if (ntile > 1) ml_tile(1, keep1, false);
      group_max(0, keep0);
      if (ntile > 1) group_max(1, keep1);
    } else if constexpr (SMALL) {
      mma_tile(first_tile, keep0);
      mma_tile(second_tile, keep1);
      group_max(0, keep0);
      if (ntile > 1) group_max(1, keep1);
    } else if constexpr (ML) {
      ml_sweep([&](int tile, f32x4_t(&acc)[4]) { group_max(tile, acc); });
    } else {
      sweep_from(first_tile, [&](int tile, f32x4_t(&acc)[4]) { group_max(tile, acc); });
    }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) gmax_s[16 * qb + r16][16 * w + 4 * g + i] = sc(gm[qb][i]);
    __syncthreads();
    {
      const int q = tid >> 2, part = tid & 3;
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = gmax_s[q][16 * part + e];
      // the m-th largest of the 64 maxima is among every lane's m largest: with m <= 8 the
      // lanes keep and merge their top 8 only
      if (m <= 8) {
        top8_of16_desc(v);
        merge8_with_lane(v, 1);
        merge8_with_lane(v, 2);
      } else {
        sort16_desc(v);
        merge16_with_lane(v, 1);
        merge16_with_lane(v, 2);
      }
      float tau = v[0];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (e == m - 1) tau = v[e];
      // long lists test raw accumulators against the least float a0 with fl(scale * a0) >= tau
      // (see below): one lane per query forms it, once
      if (part == 0) tau_s[q] = (SMALL || ML) ? tau : least_raw_bound(tau, scale);
    }
    __syncthreads();
    // sweep 2: keep the candidates at or above the bound.  The rounded product scale * a is
    // non-decreasing in a, so "scale * acc >= tau" holds exactly when acc >= a0, the least
    // float with that property: the test runs on the raw accumulators.  Each lane then
    // walks its few passing elements (rarely more than one per tile), picks each one out of
    // its sixteen accumulators with a select tree, and appends its key to the query's
    // survivor list.
    // (with at most two tiles the products are formed directly instead)
    float a0[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) a0[qb] = tau_s[16 * qb + r16];
    __syncthreads();  // every lane has read its bounds: the survivor buffer may overwrite the maxima
    auto survive = [&](int tile, const f32x4_t(&acc)[4]) {
      // in the last tile the rows past c hold scores of other chunks (or padding)
      const bool whole = (tile + 1) * 64 <= c;
      const int jb = tile * 64 + 16 * w + 4 * g;
      uint32_t bits = 0;  // bit 4 qb + i
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bits |= (((SMALL || ML) ? sc(acc[qb][i]) : acc[qb][i]) >= a0[qb] && (whole || jb + i < c)) ? (1u << (4 * qb + i))
                                                                                            : 0u;
      if (!__any(bits != 0)) return;
      // long lists: the wave parks its accumulators in LDS (four 16-byte stores a lane) and
      // each survivor reads its value back by index; short ones pick it with a select tree
      if constexpr (!SMALL) {
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) park_s[w][qb][lane] = acc[qb];
      }
      while (__any(bits != 0)) {
        if (bits != 0) {
          const int e = __builtin_ctz(bits);
          bits &= bits - 1u;
          float x;
          if constexpr (!SMALL) {
            x = reinterpret_cast<const float*>(&park_s[w][e >> 2][lane])[e & 3];
          } else {
            // element e = 4 qb + i: select on bit 0, 1 (i), then 2, 3 (qb)
            const bool b0 = (e & 1) != 0, b1 = (e & 2) != 0, b2 = (e & 4) != 0, b3 = (e & 8) != 0;
            const float y0 = b0 ? acc[0][1] : acc[0][0], y1 = b0 ? acc[0][3] : acc[0][2];
            const float y2 = b0 ? acc[1][1] : acc[1][0], y3 = b0 ? acc[1][3] : acc[1][2];
            const float y4 = b0 ? acc[2][1] : acc[2][0], y5 = b0 ? acc[2][3] : acc[2][2];
            const float y6 = b0 ? acc[3][1] : acc[3][0], y7 = b0 ? acc[3][3] : acc[3][2];
            const float z0 = b1 ? y1 : y0, z1 = b1 ? y3 : y2, z2 = b1 ? y5 : y4, z3 = b1 ? y7 : y6;
            const float u0 = b2 ? z1 : z0, u1 = b2 ? z3 : z2;
            x = b3 ? u1 : u0;
          }
          const int q = 16 * (e >> 2) + r16;
          // the key is formed while the slot is fetched, and stored without a branch: a value
          // past the slots goes to the row's padding entry (never read; the count records it)
          const uint64_t key = make_key(sc(x), jb + (e & 3));
          const int p = atomicAdd(&cnt_s[q], 1);
          surv[q][p < TK_CAP ? p : TK_CAP] = key;
        }
      }
    };
    if constexpr (SMALL) {
      survive(0, keep0);
      if (ntile > 1) survive(1, keep1);
    } else if constexpr (ML) {
      ml_sweep([&](int tile, f32x4_t(&acc)[4]) { survive(tile, acc); });
    } else {
      sweep([&](int tile, f32x4_t(&acc)[4]) { survive(tile, acc); });
    }
    __syncthreads();
    // exact top-m among the survivors by rank: a key's rank is the number of the query's
    // survivors above it (keys are distinct, so ranks are too).  The four lanes of a query take
    // its slots in turn (slot part + 4 i) and compare each with every survivor of the query;
    // each key of rank below m then goes to that row of the sorted list.  NO, the slots a lane
    // holds, follows the largest survivor count of the wavefront, so the comparisons number
    // about n * n / 4 per lane.
    {
      const int q = tid >> 2, part = tid & 3;
      const int cn = cnt_s[q];
      const int n = min(cn, TK_CAP);
      int nmax = n;
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) nmax = max(nmax, lane_xor(nmax, msk));
      // entries 0 .. NO-1 are formed and read by the variant of the same NO
      uint64_t own[TK_CAP / 4];
      int rk[TK_CAP / 4];
      auto rank_slots = [&](auto no_c) {
        constexpr int NO = decltype(no_c)::value;
#pragma unroll
        for (int i = 0; i < NO; ++i) {
          const int p = part + 4 * i;
          own[i] = p < n ? surv[q][p] : 0ull;
          rk[i] = 0;
        }
        for (int e = 0; e < nmax; ++e) {
          const uint64_t y = e < n ? surv[q][e] : 0ull;  // 0 is below every key
#pragma unroll
          for (int i = 0; i < NO; ++i) rk[i] += y > own[i] ? 1 : 0;
        }
      };
      auto place_slots = [&](auto no_c) {
        constexpr int NO = decltype(no_c)::value;
#pragma unroll
        for (int i = 0; i < NO; ++i)
          if (part + 4 * i < n && rk[i] < m) top_s[q][rk[i]] = own[i];
      };
      const int no = nmax <= 8 ? 2 : (nmax <= 16 ? 4 : (nmax <= 32 ? 8 : TK_CAP / 4));  // wavefront-uniform
      if (no == 2) rank_slots(IntC<2>{});
      else if (no == 4) rank_slots(IntC<4>{});
      else if (no == 8) rank_slots(IntC<8>{});
      else rank_slots(IntC<TK_CAP / 4>{});
      __syncthreads();  // every survivor has been read: the sorted keys overwrite the buffer
      if (no == 2) place_slots(IntC<2>{});
      else if (no == 4) place_slots(IntC<4>{});
      else if (no == 8) place_slots(IntC<8>{});
      else place_slots(IntC<TK_CAP / 4>{});
      if (part == 0 && cn > TK_CAP) atomicOr(&ovf_s, 1);
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
        auto least_below = [&](int tile, const f32x4_t(&acc)[4]) {
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
                const uint64_t key = make_key(sc(acc[qb][i]), j);
                if (key < prev && key > best) best = key;
              }
            }
            if (best) atomicMax((unsigned long long*)&best_s[q], (unsigned long long)best);
          }
        };
        // short several-landmark lists are not recomputed: the kept tiles hold them
        if constexpr (ML && SMALL) {
          least_below(0, keep0);
          if (ntile > 1) least_below(1, keep1);
        } else if constexpr (ML) {
          ml_sweep([&](int tile, f32x4_t(&acc)[4]) { least_below(tile, acc); });
        } else {
          sweep([&](int tile, f32x4_t(&acc)[4]) { least_below(tile, acc); });
        }
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

  // fusion weights and outputs: four lanes per query (slots part, part + 4, ...; the own chunk
  // in the first), the softmax statistics reduced over the four
  {
    const int q = tid >> 2, part = tid & 3;
    const float s_own = own_s[q];
    float mx = s_own;
    for (int r = part; r < m; r += 4) mx = fmaxf(mx, key_score(top_s[q][r]));
    mx = fmaxf(mx, lane_xor(mx, 1));
    mx = fmaxf(mx, lane_xor(mx, 2));
    float den = part == 0 ? __expf(s_own - mx) : 0.f;
    for (int r = part; r < m; r += 4) den += __expf(key_score(top_s[q][r]) - mx);
    den += lane_xor(den, 1);
    den += lane_xor(den, 2);
    const float inv = 1.f / den;
    const int64_t base = ((int64_t)bh * L + (int64_t)c * 64 + q) * k1;
    for (int r = part; r <= k; r += 4) {
      int ix;
      float sv, wv;
      if (r == k) {
        ix = c;
        sv = s_own;
        wv = __expf(sv - mx) * inv;
      } else if (r < m) {
        const uint64_t key = top_s[q][r];
        ix = key_index(key);
        sv = key_score(key);
        wv = __expf(sv - mx) * inv;
      } else {
        ix = -1;
        sv = -INFINITY;
        wv = 0.f;
      }
      idx[base + r] = ix;
      sel[base + r] = sv;
      if (wout) wout[base + r] = wv;
    }
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

size_t topk_workspace_bytes(int BH, int N, int d) { return (size_t)BH * klm_frag_rows(N) * d * sizeof(bf16_t); }

template <typename T, int D>
hipError_t launch_topk_t(const void* Q, const void* Klm, void* frag_ws, int32_t* idx, float* sel, float* w, int BH,
                         int L, int N, int k, float scale, hipStream_t st) {
  const T* F = nullptr;
  if (sizeof(T) == 2 && N > TK_SMALL_N) {
    const int Npad = klm_frag_rows(N);
    const int64_t pieces = (int64_t)BH * Npad * D / 8;
    HILS_LAUNCH("klm_frag", klm_frag_kernel<D>, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st,
                (const bf16_t*)Klm, (bf16_t*)frag_ws, N, Npad, pieces);
    F = (const T*)frag_ws;
  }
  dim3 grid(L / 64, BH);
  if (N <= TK_SMALL_N)
    HILS_LAUNCH("topk_select", (topk_select_kernel<T, D, true>), grid, dim3(256), 0, st, (const T*)Q, (const T*)Klm, F,
                idx, sel, w, L, N, k, scale, 1);
  else
    HILS_LAUNCH("topk_select", (topk_select_kernel<T, D, false>), grid, dim3(256), 0, st, (const T*)Q, (const T*)Klm, F,
                idx, sel, w, L, N, k, scale, 1);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_topk_ml_t(const void* Q, const void* Klm, int mlm, int32_t* idx, float* sel, float* w, int BH,
                            int L, int N, int k, float scale, hipStream_t st) {
  if (N <= TK_SMALL_N)
    HILS_LAUNCH("topk_select_ml", (topk_select_kernel<T, D, true, true>), dim3(L / 64, BH), dim3(256), 0, st,
                (const T*)Q, (const T*)Klm, (const T*)nullptr, idx, sel, w, L, N, k, scale, mlm);
  else
    HILS_LAUNCH("topk_select_ml", (topk_select_kernel<T, D, false, true>), dim3(L / 64, BH), dim3(256), 0, st,
                (const T*)Q, (const T*)Klm, (const T*)nullptr, idx, sel, w, L, N, k, scale, mlm);
  return hipGetLastError();
}

hipError_t launch_landmark_scores(int dt, int d, const void* Q, const void* Klm, float* S, int BH, int L, int N,
                                  float scale, hipStream_t st) {
  if (dt == 0) return d == 64 ? launch_landmark_scores_t<bf16_t, 64>(Q, Klm, S, BH, L, N, scale, st)
                              : launch_landmark_scores_t<bf16_t, 128>(Q, Klm, S, BH, L, N, scale, st);
  return d == 64 ? launch_landmark_scores_t<float, 64>(Q, Klm, S, BH, L, N, scale, st)
                 : launch_landmark_scores_t<float, 128>(Q, Klm, S, BH, L, N, scale, st);
}

hipError_t launch_topk_ml(int dt, int d, const void* Q, const void* Klm, int mlm, int32_t* idx, float* sel, float* w,
                          int BH, int L, int N, int k, float scale, hipStream_t st) {
  if (dt == 0) return d == 64 ? launch_topk_ml_t<bf16_t, 64>(Q, Klm, mlm, idx, sel, w, BH, L, N, k, scale, st)
                              : launch_topk_ml_t<bf16_t, 128>(Q, Klm, mlm, idx, sel, w, BH, L, N, k, scale, st);
  return d == 64 ? launch_topk_ml_t<float, 64>(Q, Klm, mlm, idx, sel, w, BH, L, N, k, scale, st)
                 : launch_topk_ml_t<float, 128>(Q, Klm, mlm, idx, sel, w, BH, L, N, k, scale, st);
}

hipError_t launch_topk(int dt, int d, const void* Q, const void* Klm, void* frag_ws, int32_t* idx, float* sel,
                       float* w, int BH, int L, int N, int k, float scale, hipStream_t st) {
  if (dt == 0) return d == 64 ? launch_topk_t<bf16_t, 64>(Q, Klm, frag_ws, idx, sel, w, BH, L, N, k, scale, st)
                              : launch_topk_t<bf16_t, 128>(Q, Klm, frag_ws, idx, sel, w, BH, L, N, k, scale, st);
  return d == 64 ? launch_topk_t<float, 64>(Q, Klm, frag_ws, idx, sel, w, BH, L, N, k, scale, st)
                 : launch_topk_t<float, 128>(Q, Klm, frag_ws, idx, sel, w, BH, L, N, k, scale, st);
}

}  // namespace hils
