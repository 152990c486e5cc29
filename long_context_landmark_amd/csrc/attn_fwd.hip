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
//                   pair writes its chunk output o_tj (bf16) and the chunk
//                   log-partition lse_tj.  The fusion weights are applied in
//                   the combine, which reads them per query row: gathered per
//                   pair here they would cost a cache line each.
//   own_combine     query-major: a workgroup takes the 64 queries of one chunk,
//                   computes their causal own-chunk attention (one 64x64 MFMA
//                   tile), adds the weighted chunk outputs of the past chunks in
//                   slot order and writes O.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

template <typename T, int D> struct alignas(16) ChunkLds {
  static constexpr int KS = D + (Elem<T>::bytes == 2 ? 8 : 4);  // row stride of K  [key][d]
  static constexpr int VS = 64 + (Elem<T>::bytes == 2 ? 4 : 4);  // row stride of V^T [d][key]
  T k[64 * KS];
  T vt[D * VS];
};

// Stage chunk rows [row0, row0+64) of K (as [key][d]) and V (as V^T [d][key]) into LDS.
// Every load is issued before the first LDS write (one memory round trip).
template <typename T, int D>
__device__ __forceinline__ void stage_chunk(ChunkLds<T, D>& s, const T* __restrict__ K, const T* __restrict__ V,
                                            int64_t row0) {
  constexpr int PER_ROW = D * Elem<T>::bytes / 16;  // 16-byte pieces per row
  constexpr int EPP = 16 / Elem<T>::bytes;           // elements per piece
  constexpr int NP = 64 * PER_ROW / 256;             // pieces per thread
  const int tid = threadIdx.x;
  int4 kv[NP], vv[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int p = tid + 256 * u;
    const int key = p / PER_ROW, e0 = (p % PER_ROW) * EPP;
    kv[u] = *reinterpret_cast<const int4*>(K + (row0 + key) * D + e0);
    vv[u] = *reinterpret_cast<const int4*>(V + (row0 + key) * D + e0);
  }
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int p = tid + 256 * u;
    const int key = p / PER_ROW, e0 = (p % PER_ROW) * EPP;
    *reinterpret_cast<int4*>(&s.k[key * ChunkLds<T, D>::KS + e0]) = kv[u];
    T vals[EPP];
    __builtin_memcpy(vals, &vv[u], 16);
#pragma unroll
    for (int e = 0; e < EPP; ++e) s.vt[(e0 + e) * ChunkLds<T, D>::VS + key] = vals[e];
  }
}

// The MFMA operand fragments of one staged chunk as a wave uses them: K rows (A operand of
// S^T = K Q^T) and V^T rows (A operand of O^T = V^T P^T).  REG = 2: both are read from LDS
// once and stay in registers for every query tile the wave runs against the chunk (64 + 64
// registers at d = 128 in bf16); REG = 1: the K fragments stay in registers and V^T is read
// from LDS at each use (fewer registers, more waves per CU); REG = 0: every use reads LDS.
template <typename T, int D, int REG> struct ChunkFrags;
template <typename T, int D> struct ChunkFrags<T, D, 2> {
  Frag<T> kf[4][D / 32];
  Frag<T> vf[D / 16][2];
  __device__ __forceinline__ void init(const ChunkLds<T, D>& s) {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) kf[cb][ks].load(&s.k[(16 * cb + r16) * ChunkLds<T, D>::KS + ks * 32 + 8 * g]);
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const T* row = &s.vt[(16 * db + r16) * ChunkLds<T, D>::VS + 32 * h + 4 * g];
        vf[db][h].load4x2(row, row + 16);
      }
  }
  __device__ __forceinline__ const Frag<T>& k(const ChunkLds<T, D>&, int cb, int ks) const { return kf[cb][ks]; }
  __device__ __forceinline__ const Frag<T>& v(const ChunkLds<T, D>&, int db, int h) const { return vf[db][h]; }
};
template <typename T, int D> struct ChunkFrags<T, D, 0> {
  __device__ __forceinline__ void init(const ChunkLds<T, D>&) {}
  __device__ __forceinline__ Frag<T> k(const ChunkLds<T, D>& s, int cb, int ks) const {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
    Frag<T> a;
    a.load(&s.k[(16 * cb + r16) * ChunkLds<T, D>::KS + ks * 32 + 8 * g]);
    return a;
  }
  __device__ __forceinline__ Frag<T> v(const ChunkLds<T, D>& s, int db, int h) const {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
    Frag<T> a;
    const T* row = &s.vt[(16 * db + r16) * ChunkLds<T, D>::VS + 32 * h + 4 * g];
    a.load4x2(row, row + 16);
    return a;
  }
};
template <typename T, int D> struct ChunkFrags<T, D, 1> {
  Frag<T> kf[4][D / 32];
  __device__ __forceinline__ void init(const ChunkLds<T, D>& s) {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) kf[cb][ks].load(&s.k[(16 * cb + r16) * ChunkLds<T, D>::KS + ks * 32 + 8 * g]);
  }
  __device__ __forceinline__ const Frag<T>& k(const ChunkLds<T, D>&, int cb, int ks) const { return kf[cb][ks]; }
  __device__ __forceinline__ Frag<T> v(const ChunkLds<T, D>& s, int db, int h) const {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
    Frag<T> a;
    const T* row = &s.vt[(16 * db + r16) * ChunkLds<T, D>::VS + 32 * h + 4 * g];
    a.load4x2(row, row + 16);
    return a;
  }
};
// K fragments in registers for the chunk kernel (the K staging area is then free for the
// output turnaround); V^T too except for bf16 at d = 128, where keeping it in LDS lets three
// workgroups share a CU; fp32 at d = 128 keeps both in LDS.
template <typename T, int D> constexpr int frags_in_regs() {
  return Elem<T>::bytes == 2 ? (D == 128 ? 1 : 2) : (D == 64 ? 2 : 0);
}

// One wave: attention of 16 query rows (given as B fragments) over the 64 keys of a chunk.
// causal_q >= 0 applies the causal mask key <= causal_q (the lane's query index inside the
// chunk).  Returns o = wt * softmax(scale * q K^T) V (4 rows of d per 16-d block; wt is the
// lane's query weight), the row's scaled maximum and its sum of exponentials relative to it.
// The exponentials are exp2 of one fused multiply-add: scale * log2(e) is folded into the
// raw scores.  16-bit inputs: they are rounded for the PV product unnormalised, and the row sums
// come from the same rounded values on the MFMA (a block of ones in place of V^T), so the
// weights that multiply V sum to one; wt / sum then scales the products.  fp32 inputs (whose
// fp32 MFMA is slow): the sums are added on the VALU and wt / sum scales the probabilities.
template <typename T, int D, int REG>
__device__ __forceinline__ void wave_chunk_attention(const ChunkLds<T, D>& s, const ChunkFrags<T, D, REG>& cf,
                                                     const Frag<T> (&qf)[D / 32], float scale, int causal_q, float wt,
                                                     f32x4_t (&o)[D / 16], float& mx, float& sum) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
  f32x4_t sc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    sc[cb] = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) mma(sc[cb], cf.k(s, cb, ks), qf[ks]);
  }
  // lane holds query r16, keys 16cb + 4g + i
  float mraw = -INFINITY;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (causal_q >= 0 && 16 * cb + 4 * g + i > causal_q) sc[cb][i] = -INFINITY;
      mraw = fmaxf(mraw, sc[cb][i]);
    }
  mraw = fmaxf(mraw, lane_xor(mraw, 16));
  mraw = fmaxf(mraw, lane_xor(mraw, 32));
  const float c2 = scale * 1.44269504088896341f;  // scale * log2(e)
  const float off = -mraw * c2;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[cb][i] = __builtin_amdgcn_exp2f(fmaf(sc[cb][i], c2, off));
  mx = scale * mraw;
  // O^T[d][q] = sum_key V^T[d][key] P^T[key][q]; element e of lane group g is key 32h + 16(e/4) + 4g + e%4
  if constexpr (Elem<T>::bytes == 4) {
    sum = 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sum += sc[cb][i];
    sum += lane_xor(sum, 16);
    sum += lane_xor(sum, 32);
    const float f = wt * __builtin_amdgcn_rcpf(sum);
    Frag<T> pf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = f * sc[2 * h + e / 4][e % 4];
      pf[h].set(pv);
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      o[db] = zero4();
#pragma unroll
      for (int h = 0; h < 2; ++h) mma(o[db], cf.v(s, db, h), pf[h]);
    }
    return;
  }
  Frag<T> pf[2], ones;
  {
    float one[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) one[e] = 1.f;
    ones.set(one);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = sc[2 * h + e / 4][e % 4];
    pf[h].set(pv);
  }
  f32x4_t rs = zero4();  // every row of it: the lane's query's sum over the 64 keys
#pragma unroll
  for (int h = 0; h < 2; ++h) mma(rs, ones, pf[h]);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    o[db] = zero4();
#pragma unroll
    for (int h = 0; h < 2; ++h) mma(o[db], cf.v(s, db, h), pf[h]);
  }
  sum = rs[0];
  const float f = wt * __builtin_amdgcn_rcpf(sum);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f * o[db];
}

template <typename T, int D, bool STREAM_OUT>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? (D == 64 ? 4 : 3) : 1) void chunk_attn_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                             const T* __restrict__ V, const int4* __restrict__ items,
                                                             const int* __restrict__ n_items,
                                                             const int* __restrict__ pairs, float* __restrict__ lse_pair,
                                                             typename PartialOf<T>::type* __restrict__ partial,
                                                             typename PartialOf<T>::type* __restrict__ trash,
                                                             float* __restrict__ trash_lse, int L, int N, int k,
                                                             int max_items, float scale, int spread) {
  using PT = typename PartialOf<T>::type;
  constexpr bool P16 = sizeof(PT) == 2;
  // A head whose query rows fit in one XCD's L2 keeps all its items on that XCD (the rows
  // gathered by its items are then read from HBM once).  Larger heads are spread over all
  // XCDs, head after head, so the query rows of the few heads in flight stay in the
  // memory-side cache.
  int item, bh;
  if (spread) {
    item = blockIdx.x;
    bh = blockIdx.y;
  } else {
    xcd_map(item, bh);
  }
  // the item (chunk, pair range) and the item count are read together; items past the count
  // hold stale data and are discarded
  const int4 it = items[(int64_t)bh * max_items + item];
  if (item >= n_items[bh]) return;
  const int j = it.x;
  const int p0 = it.y, p1 = it.z;
  __shared__ ChunkLds<T, D> s;
  const int tid = threadIdx.x, w_ = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const int* pl = pairs + (int64_t)bh * L * k;
  const T* Qb = Q + (int64_t)bh * L * D;
  // Software pipeline over 64-pair tiles with three register sets used in turn, so no loaded
  // value is ever copied: while tile i runs on one set, the query rows of
  // tiles i+1 and i+2 are in flight in the other two and the pair entries of tile i+3 are
  // read.  Loads are unconditional (clamped to valid rows; rows of absent pairs are computed
  // and dropped) so that every wait covers exactly the data about to be used.
  // bf16 query rows of d = 128 are gathered a quad per row and assembled into fragments
  // with a lane permutation just before use (the pair entry of the row a lane loads is read
  // for it).  At d = 64 the direct fragment loads measured faster.
  constexpr bool QUAD = sizeof(T) == 2 && D == 128;
  const int qrow = QUAD ? quad_row(lane) : r16, qpc = QUAD ? quad_piece(lane) : g;
  auto pair_raw = [&](int base) { return pl[min(base + 16 * w_ + r16, p1 - 1)]; };
  auto pair_ok = [&](int base) { return base + 16 * w_ + r16 < p1; };
  auto gat_raw = [&](int base) { return pl[min(base + 16 * w_ + qrow, p1 - 1)]; };
  auto gat_ok = [&](int base) { return base + 16 * w_ + qrow < p1; };
  auto load_q = [&](int pe, Frag<T>(&qf)[D / 32]) {
    const int64_t t = pe >= 0 ? (pe >> 5) : 0;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[ks].load(Qb + t * D + ks * 32 + 8 * qpc);
  };
  ChunkFrags<T, D, frags_in_regs<T, D>()> cf;
  // Results go to the pairs' own positions in the list, so a tile's 64 rows are consecutive.
  // When all partial rows together exceed the memory-side cache they are stored as streaming
  // (non-temporal) data, which keeps the cache for the gathered query rows; smaller sets stay
  // cached for the combine, which reads them right after.
  // With the chunk's fragments in registers the staging LDS is free after they are read: each
  // wave then turns its 16 output rows around there and stores them as whole rows (16 bytes a
  // lane, 1 KiB a store).  Rows of absent pairs go to a scratch row: every lane stores, so
  // the waits on the loads of the next tiles can count the stores.
  constexpr bool ROWS = frags_in_regs<T, D>() > 0;
  constexpr int EPV = 16 / (int)sizeof(PT);         // partial elements per 16-byte piece
  constexpr int RSB = D + (P16 ? 8 : 4);             // row stride of the turnaround buffer (elements)
  PT* rowbuf = reinterpret_cast<PT*>(&s) + w_ * 16 * RSB;
  static_assert(!ROWS || 4 * 16 * RSB * (int)sizeof(PT) <= 64 * ChunkLds<T, D>::KS * (int)sizeof(T),
                "turnaround buffer fits the K staging area");
  auto tile = [&](const Frag<T>(&qf)[D / 32], int pe, int base) {
    Frag<T> qx[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qx[ks] = qf[ks];
      if constexpr (QUAD) frag_from_quads(qx[ks], lane);
    }
    f32x4_t o[D / 16];
    float mx, sum;
    wave_chunk_attention(s, cf, qx, scale, -1, 1.f, o, mx, sum);
    const bool ok = pe >= 0;
    const int64_t prow = (int64_t)bh * L * k + base + 16 * w_ + r16;
    if constexpr (ROWS) {
      constexpr int PPR = D / EPV, RPI = 64 / PPR;  // 16-byte pieces per row, rows per store
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        if constexpr (P16)
          *reinterpret_cast<uint2*>(rowbuf + r16 * RSB + 16 * db + 4 * g) =
              make_uint2(pack_bf16x2(o[db][0], o[db][1]), pack_bf16x2(o[db][2], o[db][3]));
        else
          *reinterpret_cast<f32x4_t*>(rowbuf + r16 * RSB + 16 * db + 4 * g) = o[db];
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < 16 / RPI; ++it) {
        const int row = it * RPI + lane / PPR, pc = lane % PPR;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(rowbuf + row * RSB + EPV * pc);
        const int pidx = base + 16 * w_ + row;
        PT* dst = pidx < p1 ? partial + ((int64_t)bh * L * k + pidx) * D : trash;
        if constexpr (STREAM_OUT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst + EPV * pc));
        else *reinterpret_cast<u32x4_t*>(dst + EPV * pc) = v;
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      PT* dst = ok ? partial + prow * D : trash;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        if constexpr (P16) {
          const uint2 v2 = make_uint2(pack_bf16x2(o[db][0], o[db][1]), pack_bf16x2(o[db][2], o[db][3]));
          *reinterpret_cast<uint2*>(dst + 16 * db + 4 * g) = v2;
        } else {
          *reinterpret_cast<f32x4_t*>(dst + 16 * db + 4 * g) = o[db];
        }
      }
    }
    // the four lane groups hold the same row statistics
    *(ok ? lse_pair + prow : trash_lse) = mx + __logf(sum);
  };
  Frag<T> q0[D / 32], q1[D / 32], q2[D / 32];
  int pe0 = pair_ok(p0) ? pair_raw(p0) : -1;
  int pe1 = pair_ok(p0 + 64) ? pair_raw(p0 + 64) : -1;
  int pe2;
  load_q(gat_ok(p0) ? gat_raw(p0) : -1, q0);
  load_q(gat_ok(p0 + 64) ? gat_raw(p0 + 64) : -1, q1);
  int raw = pair_raw(p0 + 128), graw = gat_raw(p0 + 128);
  stage_chunk<T, D>(s, K + (int64_t)bh * L * D, V + (int64_t)bh * L * D, (int64_t)j * 64);
  __syncthreads();
  cf.init(s);
  if constexpr (ROWS) __syncthreads();  // every wave holds its fragments: the staging LDS is reused
  // one step: resolve the entry of tile base+128, start its loads into the free set, read the
  // entry of tile base+192, run tile base
#define HILS_FWD_STEP(QU, PU, QF, PF)                           \
  PF = pair_ok(base + 128) ? raw : -1;                         \
  load_q(gat_ok(base + 128) ? graw : -1, QF);                  \
  raw = pair_raw(base + 192);                                  \
  graw = gat_raw(base + 192);                                  \
  tile(QU, PU, base);                                          \
  base += 64;                                                  \
  if (base >= p1) break;
  for (int base = p0;;) {
    HILS_FWD_STEP(q0, pe0, q2, pe2)
    HILS_FWD_STEP(q1, pe1, q0, pe0)
    HILS_FWD_STEP(q2, pe2, q1, pe1)
  }
#undef HILS_FWD_STEP
}

// Per query chunk: the causal own-chunk tile on MFMA, then the fusion sum in row layout.
// The weighted own output goes through LDS into rows; each thread then owns 16-byte pieces
// of output rows and adds the same piece of the query's chunk outputs, each times its fusion
// weight; chunk_attn_fwd stored them at the pairs' list positions (pos_of): every partial
// row is read as whole 128-byte lines, and O and lse are written row by row.
template <typename T, int D>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? (D == 64 ? 5 : 3) : 1) void own_combine_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                          const T* __restrict__ V, const int* __restrict__ pos_of,
                                                          const float* __restrict__ w,
                                                          const typename PartialOf<T>::type* __restrict__ partial,
                                                          const float* __restrict__ lse_pair, T* __restrict__ O,
                                                          float* __restrict__ lse, int L, int N, int k, float scale) {
  using PT = typename PartialOf<T>::type;
  constexpr int VPP = (int)sizeof(PT) / 2;  // 16-byte loads per 8-element piece
  constexpr int RS = D + 4;         // row stride of the output rows in LDS (floats)
  constexpr int PPR = D / 8;        // 8-element pieces per row
  constexpr int NI = 64 * PPR / 256;  // pieces per thread
  int c, bh;
  xcd_map(c, bh);
  __shared__ union {
    ChunkLds<T, D> s;
    float orow[64 * RS];
  } u;
  __shared__ int pos_s[64][16];
  __shared__ float w_s[64][16];
  __shared__ float own_lse[64];
  const int tid = threadIdx.x, w_ = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const int qi = 16 * w_ + r16;  // query inside the chunk (MFMA layout)
  const int64_t row0 = (int64_t)bh * L + (int64_t)c * 64;
  const int k1 = k + 1;
  // requested before the first wait: query rows, own weight, the list positions of the
  // query chunk's pairs, the chunk's keys and values
  Frag<T> qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qf[ks].load(Q + (row0 + qi) * D + ks * 32 + 8 * g);
  const float w_own = w[(row0 + qi) * k1 + k];
  int pv[4];
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;  // (query, slot) = (e / 16, e % 16); slots >= k are unused
    pv[i] = (e % 16) < k ? pos_of[(row0 + e / 16) * k + (e % 16)] : -1;
    wv[i] = (e % 16) < k ? w[(row0 + e / 16) * k1 + (e % 16)] : 0.f;
  }
  stage_chunk<T, D>(u.s, K + (int64_t)bh * L * D, V + (int64_t)bh * L * D, (int64_t)c * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pos_s[(tid + 256 * i) / 16][(tid + 256 * i) % 16] = pv[i];
    w_s[(tid + 256 * i) / 16][(tid + 256 * i) % 16] = wv[i];
  }
  __syncthreads();
  f32x4_t o[D / 16];
  float mx, sum;
  ChunkFrags<T, D, 0> cf;  // one tile: the fragments are read once either way
  wave_chunk_attention(u.s, cf, qf, scale, qi, w_own, o, mx, sum);
  __syncthreads();  // every wave is done with the keys and values: the rows reuse their space
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) u.orow[qi * RS + 16 * db + 4 * g + i] = o[db][i];
  if (g == 0) own_lse[qi] = mx + __logf(sum);
  __syncthreads();
  const int64_t pbase = (int64_t)bh * L * k;
  float acc[NI][8];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int e = tid + 256 * it, q = e / PPR, pc = e % PPR;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[it][x] = u.orow[q * RS + 8 * pc + x];
  }
  // partial pieces of SB slots for every owned piece are in flight together; a slot whose
  // position is -1 reads row 0 of the head's list and is dropped
  constexpr int SB = (NI == 2 ? 8 : 4) / VPP;
  const int m = min(k, 16);
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += SB) {
    if (r0 >= m) break;
    u32x4_t v[NI][SB][VPP];
    bool kept[NI][SB];
    float wt[NI][SB];
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int e = tid + 256 * it, q = e / PPR, pc = e % PPR;
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const int p = pos_s[q][r0 + sb];
        kept[it][sb] = p >= 0;
        wt[it][sb] = w_s[q][r0 + sb];
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(partial + (pbase + max(p, 0)) * D + 8 * pc);
#pragma unroll
        for (int h = 0; h < VPP; ++h) v[it][sb][h] = __builtin_nontemporal_load(src + h);
      }
    }
#pragma unroll
    for (int it = 0; it < NI; ++it)
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        float pv[8];
        if constexpr (VPP == 1) {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            pv[2 * x] = __uint_as_float(v[it][sb][0][x] << 16);
            pv[2 * x + 1] = __uint_as_float(v[it][sb][0][x] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int x = 0; x < 8; ++x) pv[x] = __uint_as_float(v[it][sb][x / 4][x % 4]);
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[it][x] += kept[it][sb] ? wt[it][sb] * pv[x] : 0.f;
      }
  }
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int e = tid + 256 * it, q = e / PPR, pc = e % PPR;
#pragma unroll
    for (int x = 0; x < 8; ++x) Elem<T>::store(O, (row0 + q) * D + 8 * pc + x, acc[it][x]);
  }
  if (lse) {
    for (int e = tid; e < 64 * k1; e += 256) {
      const int q = e / k1, r = e % k1;
      float v = own_lse[q];
      if (r < k) {
        const int p = pos_s[q][r];
        v = p >= 0 ? lse_pair[pbase + p] : -INFINITY;
      }
      lse[row0 * k1 + e] = v;
    }
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
static hipError_t chunk_attn_t(const void* Q, const void* K, const void* V, const RouteBufs& rb, float* lse,
                               void* partial_v, void* trash_v, float* trash_lse, int BH, int L, int N, int k,
                               float scale, hipStream_t st) {
  using PT = typename PartialOf<T>::type;
  PT* partial = (PT*)partial_v;
  PT* trash = (PT*)trash_v;
  const int spread = (int64_t)L * D * sizeof(T) > L2_BYTES_PER_XCD;
  if ((int64_t)BH * L * k * D * (int64_t)sizeof(PT) > MALL_BYTES)
    HILS_LAUNCH("chunk_attn_fwd", (chunk_attn_fwd_kernel<T, D, true>), dim3(rb.max_items, BH), dim3(256), 0, st,
                (const T*)Q, (const T*)K, (const T*)V, rb.items, rb.n_items, rb.pairs, lse, partial,
                trash, trash_lse, L, N, k, rb.max_items, scale, spread);
  else
    HILS_LAUNCH("chunk_attn_fwd", (chunk_attn_fwd_kernel<T, D, false>), dim3(rb.max_items, BH), dim3(256), 0, st,
                (const T*)Q, (const T*)K, (const T*)V, rb.items, rb.n_items, rb.pairs, lse, partial,
                trash, trash_lse, L, N, k, rb.max_items, scale, spread);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t own_combine_t(const void* Q, const void* K, const void* V, const int* pos_of, const float* w,
                                const void* partial, const float* lse_pair, void* O, float* lse, int BH, int L,
                                int N, int k, float scale, hipStream_t st) {
  HILS_LAUNCH("own_combine", (own_combine_kernel<T, D>), dim3(N, BH), dim3(256), 0, st, (const T*)Q, (const T*)K,
              (const T*)V, pos_of, w, (const typename PartialOf<T>::type*)partial, lse_pair, (T*)O, lse, L, N, k,
              scale);
  return hipGetLastError();
}

hipError_t launch_chunk_attn_fwd(int dt, int d, const void* Q, const void* K, const void* V, const RouteBufs& rb,
                                 float* lse, void* partial, void* trash, float* trash_lse,
                                 int BH, int L, int N, int k, float scale, hipStream_t st) {
  if (dt == 0)
    return d == 64 ? chunk_attn_t<bf16_t, 64>(Q, K, V, rb, lse, partial, trash, trash_lse, BH, L, N, k, scale, st)
                   : chunk_attn_t<bf16_t, 128>(Q, K, V, rb, lse, partial, trash, trash_lse, BH, L, N, k, scale, st);
  return d == 64 ? chunk_attn_t<float, 64>(Q, K, V, rb, lse, partial, trash, trash_lse, BH, L, N, k, scale, st)
                 : chunk_attn_t<float, 128>(Q, K, V, rb, lse, partial, trash, trash_lse, BH, L, N, k, scale, st);
}

hipError_t launch_own_combine(int dt, int d, const void* Q, const void* K, const void* V, const int* pos_of,
                              const float* w, const void* partial, const float* lse_pair, void* O, float* lse,
                              int BH, int L, int N, int k, float scale, hipStream_t st) {
  if (dt == 0)
    return d == 64 ? own_combine_t<bf16_t, 64>(Q, K, V, pos_of, w, partial, lse_pair, O, lse, BH, L, N, k, scale, st)
                   : own_combine_t<bf16_t, 128>(Q, K, V, pos_of, w, partial, lse_pair, O, lse, BH, L, N, k, scale, st);
  return d == 64 ? own_combine_t<float, 64>(Q, K, V, pos_of, w, partial, lse_pair, O, lse, BH, L, N, k, scale, st)
                 : own_combine_t<float, 128>(Q, K, V, pos_of, w, partial, lse_pair, O, lse, BH, L, N, k, scale, st);
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
