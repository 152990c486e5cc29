// Per-chunk attention and score-weighted fusion (HiLS attention, steps 3-4).
//
// Passages defining the operation:
//   "Hierarchical Sparse Attention Done Right" abstract (chatpaper page):
//   every query attends to each retrieved chunk on its own, and the per-chunk
//   results are fused according to the chunk retrieval scores;
//   ai-feeds summary, "Method" > "Key modules" item 2 (ordinary attention of
//   the query with each retrieved chunk's keys and values, then a fusion
//   weighted by the retrieval scores) and item 1 (chunk-level softmax);
//   paper.oopus.info review, section 2 (in-chunk attention, weighted fusion).
// Fixed here: both softmax levels use scale 1/sqrt(d) by default; the fusion
// softmax runs over the selected set only; the own chunk is attended causally.
//
// Two kernels:
//   chunk_attn_fwd  chunk-major: a workgroup holds one past chunk's K and V^T in
//                   LDS and runs 64-query tiles of the queries that selected it
//                   (gathered through the routing lists) on bf16 MFMA.  Each
//                   pair writes its pre-weighted partial w_tj * o_tj (bf16) and
//                   the chunk log-partition lse_tj.
//   own_combine     query-major: a workgroup takes the 64 queries of one chunk,
//                   computes their causal own-chunk attention (one 64x64 MFMA
//                   tile), adds the partials of the past chunks in slot order
//                   and writes O.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

template <typename T, int D> struct ChunkLds {
  static constexpr int KS = D + (Elem<T>::bytes == 2 ? 8 : 4);  // row stride of K  [key][d]
  static constexpr int VS = 64 + (Elem<T>::bytes == 2 ? 4 : 4);  // row stride of V^T [d][key]
  T k[64 * KS];
  T vt[D * VS];
};

// Stage chunk rows [row0, row0+64) of K (as [key][d]) and V (as V^T [d][key]) into LDS.
template <typename T, int D>
__device__ __forceinline__ void stage_chunk(ChunkLds<T, D>& s, const T* __restrict__ K, const T* __restrict__ V,
                                            int64_t row0) {
  constexpr int PER_ROW = D * Elem<T>::bytes / 16;  // 16-byte pieces per row
  constexpr int EPP = 16 / Elem<T>::bytes;           // elements per piece
  const int tid = threadIdx.x;
  for (int p = tid; p < 64 * PER_ROW; p += 256) {
    const int key = p / PER_ROW, e0 = (p % PER_ROW) * EPP;
    const int4 kv = *reinterpret_cast<const int4*>(K + (row0 + key) * D + e0);
    *reinterpret_cast<int4*>(&s.k[key * ChunkLds<T, D>::KS + e0]) = kv;
    const int4 vv = *reinterpret_cast<const int4*>(V + (row0 + key) * D + e0);
    T vals[EPP];
    __builtin_memcpy(vals, &vv, 16);
#pragma unroll
    for (int e = 0; e < EPP; ++e) s.vt[(e0 + e) * ChunkLds<T, D>::VS + key] = vals[e];
  }
}

// One wave: attention of 16 query rows (given as B fragments) over the 64 keys in LDS.
// mask_q >= 0 applies the causal mask key <= mask_q + (query index inside the block);
// returns o (unnormalised, 4 rows of d per 16-d block), the row max and the row sum.
template <typename T, int D>
__device__ __forceinline__ void wave_chunk_attention(const ChunkLds<T, D>& s, const Frag<T> (&qf)[D / 32],
                                                     float scale, int causal_q, f32x4_t (&o)[D / 16], float& mx,
                                                     float& sum) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  f32x4_t sc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    sc[cb] = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      Frag<T> a;
      a.load(&s.k[(16 * cb + r16) * ChunkLds<T, D>::KS + ks * 32 + 8 * g]);
      mma(sc[cb], a, qf[ks]);
    }
  }
  // lane holds query r16, keys 16cb + 4g + i
  mx = -INFINITY;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = scale * sc[cb][i];
      if (causal_q >= 0 && 16 * cb + 4 * g + i > causal_q) v = -INFINITY;
      sc[cb][i] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, lane_xor(mx, 16));
  mx = fmaxf(mx, lane_xor(mx, 32));
  sum = 0.f;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __expf(sc[cb][i] - mx);
      sc[cb][i] = p;
      sum += p;
    }
  sum += lane_xor(sum, 16);
  sum += lane_xor(sum, 32);
  // O^T[d][q] = sum_key V^T[d][key] P^T[key][q]; element e of lane group g is key 32h + 16(e/4) + 4g + e%4
  Frag<T> pf[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = sc[2 * h + e / 4][e % 4];
    pf[h].set(pv);
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    o[db] = zero4();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Frag<T> vf;
      const T* row = &s.vt[(16 * db + r16) * ChunkLds<T, D>::VS + 32 * h + 4 * g];
      vf.load4x2(row, row + 16);
      mma(o[db], vf, pf[h]);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_attn_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                             const T* __restrict__ V, const int* __restrict__ chunk_off,
                                                             const int4* __restrict__ items,
                                                             const int* __restrict__ n_items,
                                                             const int* __restrict__ pairs,
                                                             const float* __restrict__ w, float* __restrict__ lse,
                                                             uint16_t* __restrict__ partial, int L, int N, int k,
                                                             int max_items, int ppi, float scale) {
  int item, bh;
  xcd_map(item, bh);
  // the item (chunk, pair range) and the item count are read together; items past the count
  // hold stale data and are discarded
  const int4 it = items[(int64_t)bh * max_items + item];
  if (item >= n_items[bh]) return;
  const int j = it.x;
  const int p0 = it.y, p1 = it.z;
  (void)chunk_off;
  (void)ppi;
  __shared__ ChunkLds<T, D> s;
  const int tid = threadIdx.x, w_ = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const int* pl = pairs + (int64_t)bh * L * k;
  const T* Qb = Q + (int64_t)bh * L * D;
  const int k1 = k + 1;
  // software pipeline over 64-pair tiles: pair entries two tiles ahead, query rows one tile ahead
  auto pair_at = [&](int base) { const int pidx = base + 16 * w_ + r16; return pidx < p1 ? pl[pidx] : -1; };
  auto load_q = [&](int pe, Frag<T>(&qf)[D / 32]) {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      if (pe >= 0) qf[ks].load(Qb + (int64_t)(pe >> 5) * D + ks * 32 + 8 * g);
      else qf[ks].zero();
    }
  };
  int pe_cur = pair_at(p0), pe_nxt = pair_at(p0 + 64);
  Frag<T> q_cur[D / 32], q_nxt[D / 32];
  load_q(pe_cur, q_cur);
  stage_chunk<T, D>(s, K + (int64_t)bh * L * D, V + (int64_t)bh * L * D, (int64_t)j * 64);
  __syncthreads();
  for (int base = p0; base < p1; base += 64) {
    const bool more = base + 64 < p1;
    if (more) load_q(pe_nxt, q_nxt);
    const int pe_after = (base + 128 < p1) ? pair_at(base + 128) : -1;
    f32x4_t o[D / 16];
    float mx, sum;
    wave_chunk_attention<T, D>(s, q_cur, scale, -1, o, mx, sum);
    if (pe_cur >= 0) {
      const int t = pe_cur >> 5, r = pe_cur & 31;
      const int64_t prow = (int64_t)bh * L + t;
      const float f = w[prow * k1 + r] / sum;
      uint16_t* dst = partial + (prow * k + r) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        u16x4_t v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = f32_to_bf16(f * o[db][i]);
        *reinterpret_cast<u16x4_t*>(dst + 16 * db + 4 * g) = v4;
      }
      if (lse && g == 0) lse[prow * k1 + r] = mx + __logf(sum);
    }
    if (more) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) q_cur[ks] = q_nxt[ks];
    }
    pe_cur = pe_nxt;
    pe_nxt = pe_after;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void own_combine_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                          const T* __restrict__ V, const int32_t* __restrict__ idx,
                                                          const float* __restrict__ w,
                                                          const uint16_t* __restrict__ partial, T* __restrict__ O,
                                                          float* __restrict__ lse, int L, int N, int k, float scale) {
  int c, bh;
  xcd_map(c, bh);
  __shared__ ChunkLds<T, D> s;
  stage_chunk<T, D>(s, K + (int64_t)bh * L * D, V + (int64_t)bh * L * D, (int64_t)c * 64);
  __syncthreads();
  const int tid = threadIdx.x, w_ = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const int qi = 16 * w_ + r16;  // query inside the chunk
  const int64_t prow = (int64_t)bh * L + (int64_t)c * 64 + qi;
  Frag<T> qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qf[ks].load(Q + prow * D + ks * 32 + 8 * g);
  f32x4_t o[D / 16];
  float mx, sum;
  wave_chunk_attention<T, D>(s, qf, scale, qi, o, mx, sum);
  const int k1 = k + 1;
  const int m = min(k, c);
  const float f = w[prow * k1 + k] / sum;
  float acc[D / 16][4];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[db][i] = 0.f;
  // kept-slot flags first, then the partial rows four slots at a time (loads in flight together)
  bool kept[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) kept[r] = r < m && idx[prow * k1 + r] >= 0;
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += 4) {
    if (r0 >= m) break;
    u16x4_t v[4][D / 16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint16_t* src = partial + (prow * k + r0 + u) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        if (kept[r0 + u]) v[u][db] = *reinterpret_cast<const u16x4_t*>(src + 16 * db + 4 * g);
        else v[u][db] = u16x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[db][i] += bf16_to_f32(v[u][db][i]);
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) Elem<T>::store(O, prow * D + 16 * db + 4 * g + i, acc[db][i] + f * o[db][i]);
  if (lse && g == 0) {
    lse[prow * k1 + k] = mx + __logf(sum);
    for (int r = 0; r < k; ++r)
      if (r >= m || idx[prow * k1 + r] < 0) lse[prow * k1 + r] = -INFINITY;
  }
}

// Scores and fusion weights of a caller-given selection: one thread per query row.
template <typename T>
__global__ __launch_bounds__(256) void fixed_selection_kernel(const T* __restrict__ Q, const T* __restrict__ Klm,
                                                              const int32_t* __restrict__ idx, float* __restrict__ sel,
                                                              float* __restrict__ w, int64_t rows, int L, int N,
                                                              int d, int k, float scale) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int64_t bh = row / L;
  const int k1 = k + 1;
  float mx = -INFINITY;
  for (int r = 0; r < k1; ++r) {
    const int j = idx[row * k1 + r];
    float s = -INFINITY;
    if (j >= 0 && j < N) {
      float dot = 0.f;
      for (int e = 0; e < d; ++e) dot += Elem<T>::to_f32(Q, row * d + e) * Elem<T>::to_f32(Klm, (bh * N + j) * d + e);
      s = scale * dot;
    }
    sel[row * k1 + r] = s;
    mx = fmaxf(mx, s);
  }
  float den = 0.f;
  for (int r = 0; r < k1; ++r) den += idx[row * k1 + r] >= 0 ? __expf(sel[row * k1 + r] - mx) : 0.f;
  for (int r = 0; r < k1; ++r)
    if (w) w[row * k1 + r] = idx[row * k1 + r] >= 0 ? __expf(sel[row * k1 + r] - mx) / den : 0.f;
}

template <typename T, int D>
static hipError_t chunk_attn_t(const void* Q, const void* K, const void* V, const RouteBufs& rb, const float* w,
                               float* lse, uint16_t* partial, int BH, int L, int N, int k, float scale,
                               hipStream_t st) {
  HILS_LAUNCH("chunk_attn_fwd", (chunk_attn_fwd_kernel<T, D>), dim3(rb.max_items, BH), dim3(256), 0, st, (const T*)Q,
                     (const T*)K, (const T*)V, rb.chunk_off, rb.items, rb.n_items, rb.pairs, w, lse, partial, L, N,
                     k, rb.max_items, rb.pairs_per_item, scale);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t own_combine_t(const void* Q, const void* K, const void* V, const int32_t* idx, const float* w,
                                const uint16_t* partial, void* O, float* lse, int BH, int L, int N, int k, float scale,
                                hipStream_t st) {
  HILS_LAUNCH("own_combine", (own_combine_kernel<T, D>), dim3(N, BH), dim3(256), 0, st, (const T*)Q, (const T*)K,
                     (const T*)V, idx, w, partial, (T*)O, lse, L, N, k, scale);
  return hipGetLastError();
}

hipError_t launch_chunk_attn_fwd(int dt, int d, const void* Q, const void* K, const void* V, const RouteBufs& rb,
                                 const float* w, float* lse, uint16_t* partial, int BH, int L, int N, int k,
                                 float scale, hipStream_t st) {
  if (dt == 0) return d == 64 ? chunk_attn_t<bf16_t, 64>(Q, K, V, rb, w, lse, partial, BH, L, N, k, scale, st)
                              : chunk_attn_t<bf16_t, 128>(Q, K, V, rb, w, lse, partial, BH, L, N, k, scale, st);
  return d == 64 ? chunk_attn_t<float, 64>(Q, K, V, rb, w, lse, partial, BH, L, N, k, scale, st)
                 : chunk_attn_t<float, 128>(Q, K, V, rb, w, lse, partial, BH, L, N, k, scale, st);
}

hipError_t launch_own_combine(int dt, int d, const void* Q, const void* K, const void* V, const int32_t* idx,
                              const float* w, const uint16_t* partial, void* O, float* lse, int BH, int L, int N, int k,
                              float scale, hipStream_t st) {
  if (dt == 0) return d == 64 ? own_combine_t<bf16_t, 64>(Q, K, V, idx, w, partial, O, lse, BH, L, N, k, scale, st)
                              : own_combine_t<bf16_t, 128>(Q, K, V, idx, w, partial, O, lse, BH, L, N, k, scale, st);
  return d == 64 ? own_combine_t<float, 64>(Q, K, V, idx, w, partial, O, lse, BH, L, N, k, scale, st)
                 : own_combine_t<float, 128>(Q, K, V, idx, w, partial, O, lse, BH, L, N, k, scale, st);
}

hipError_t launch_fixed_selection(int dt, int d, const void* Q, const void* Klm, const int32_t* idx, float* sel,
                                  float* w, int BH, int L, int N, int k, float scale, hipStream_t st) {
  const int64_t rows = (int64_t)BH * L;
  const dim3 grid((unsigned)((rows + 255) / 256));
  if (dt == 0)
    HILS_LAUNCH("fixed_selection", fixed_selection_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)Q, (const bf16_t*)Klm,
                       idx, sel, w, rows, L, N, d, k, scale);
  else
    HILS_LAUNCH("fixed_selection", fixed_selection_kernel<float>, grid, dim3(256), 0, st, (const float*)Q, (const float*)Klm, idx,
                       sel, w, rows, L, N, d, k, scale);
  return hipGetLastError();
}

}  // namespace hils
