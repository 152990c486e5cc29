// Backward pass of HiLS attention with the selection held fixed.
//
// Passages: "Hierarchical Sparse Attention Done Right" abstract (chatpaper
// page): the retrieval scores enter the forward computation, so they are
// trained by the language-modelling loss, which gives native sparse training;
// ai-feeds summary, "Method" > "Key modules" items 1 and 3 and "Output &
// training" (the selection scores get gradients through the fused output).
// The top-k choice itself is a hard, constant selection.
//
// For query t with upstream gradient g = dO_t, kept chunks j (weights w_j,
// per-chunk outputs o_j, in-chunk probabilities p_i):
//   D_j = g.o_j,  D = g.o_t = sum_j w_j D_j,  ds_j = w_j (D_j - D)
//   da_i = w_j p_i (g.v_i - D_j)
//   dV_i += w_j p_i g     dK_i += scale da_i q_t     dQ_t += scale da_i k_i
//   dQ_t += scale ds_j Klm_j                          dKlm_j += scale ds_j q_t
// D is formed exactly as sum_j w_j D_j from the per-chunk D_j, so that the
// fusion gradients ds_j sum to zero for every query as they do in the maths
// (a D taken from the rounded forward output would not).
//
// Kernels:
//   chunk_bwd    one workgroup per chunk j: its own-chunk tile (the 64 queries
//                of chunk j, causal) and then the tiles of the queries that
//                selected j (routing lists, ascending (t, slot)).  dK_j and
//                dV_j accumulate inside the workgroup in a fixed order, so they
//                are written once, without atomics, and bit-for-bit
//                reproducible.  Every pair writes its in-chunk dQ contribution
//                and D_j to per-(query, slot) buffers.
//   dq_reduce    per query: D, ds_j, and dQ_t = sum over slots (slot order) of
//                the in-chunk parts plus scale * sum_j ds_j Klm_j; ds is kept.
//   klm_bwd      one workgroup per chunk j: dKlm_j = scale * sum ds_tj q_t over
//                the chunk's pairs in routing order.
#include "hils_device.h"
#include "hils_launch.h"
#include "lf_means.h"

namespace hils {

// 16-bit inputs (TR): the tile's Q, dO, w P and dA are staged row-major by tile query (16- and
// 8-byte stores) and the dV, dK operands are read through transposing LDS loads; fp32 inputs
// stage them transposed, element by element.
// SPLIT (fp32 at d = 128, whose seven tiles would take 207 KB): dO and w P are staged and the dV
// products formed first, then Q and dA take the same buffers for the dK products.
template <typename T, int D> struct alignas(16) BwdLds {
  static constexpr bool TR = Elem<T>::bytes == 2;
  static constexpr bool SPLIT = !TR && D == 128;
  static constexpr int KS = D + (Elem<T>::bytes == 2 ? 8 : 4);   // rows indexed by key, d inside
  static constexpr int TS = 64 + (Elem<T>::bytes == 2 ? 8 : 4);  // rows of 64 (keys or tile queries)
  static constexpr int QS = D + 8;                               // TR: rows of D (tile query, d)
  T k[64 * KS];
  T v[64 * KS];
  static constexpr int UNUSED = 16 / (int)sizeof(T);  // one 16-byte piece keeps the next array aligned
  T kt[D * TS];                                // K^T   [d][key]
  T qt[TR ? 64 * QS : D * TS];                 // TR: Q  [tile query][d];   fp32: Q^T  [d][tile query]
  T gt_[SPLIT ? UNUSED : (TR ? 64 * QS : D * TS)];  // TR: dO [tile query][d];   fp32: dO^T [d][tile query]
  T pt[64 * TS];                               // TR: w P [tile query][key]; fp32: (w P)^T [key][tile query]
  T dat_[SPLIT ? UNUSED : 64 * TS];            // TR: dA  [tile query][key]; fp32: dA^T  [key][tile query]
  __device__ __forceinline__ T* gt() { return SPLIT ? qt : gt_; }
  __device__ __forceinline__ const T* gt() const { return SPLIT ? qt : gt_; }
  __device__ __forceinline__ T* dat() { return SPLIT ? pt : dat_; }
  __device__ __forceinline__ const T* dat() const { return SPLIT ? pt : dat_; }
};

// The chunk's K and V rows as A fragments of S^T = K Q^T and dP^T = V dO^T: held in registers
// for every tile of the chunk (bf16 at d = 64: 64 registers) or read from LDS at each use.
template <typename T, int D, bool REG> struct KVFrags;
template <typename T, int D> struct KVFrags<T, D, true> {
  Frag<T> kf[4][D / 32], vf[4][D / 32];
  __device__ __forceinline__ void init(const BwdLds<T, D>& s) {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        kf[cb][ks].load(&s.k[(16 * cb + r16) * BwdLds<T, D>::KS + ks * 32 + 8 * g]);
        vf[cb][ks].load(&s.v[(16 * cb + r16) * BwdLds<T, D>::KS + ks * 32 + 8 * g]);
      }
  }
  __device__ __forceinline__ const Frag<T>& k(const BwdLds<T, D>&, int cb, int ks) const { return kf[cb][ks]; }
  __device__ __forceinline__ const Frag<T>& v(const BwdLds<T, D>&, int cb, int ks) const { return vf[cb][ks]; }
};
template <typename T, int D> struct KVFrags<T, D, false> {
  __device__ __forceinline__ void init(const BwdLds<T, D>&) {}
  __device__ __forceinline__ Frag<T> k(const BwdLds<T, D>& s, int cb, int ks) const {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
    Frag<T> a;
    a.load(&s.k[(16 * cb + r16) * BwdLds<T, D>::KS + ks * 32 + 8 * g]);
    return a;
  }
  __device__ __forceinline__ Frag<T> v(const BwdLds<T, D>& s, int cb, int ks) const {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
    Frag<T> a;
    a.load(&s.v[(16 * cb + r16) * BwdLds<T, D>::KS + ks * 32 + 8 * g]);
    return a;
  }
};

// bf16 at d = 64: two workgroups per CU, whose 256 registers a lane then all sit in the vector
// file (unbounded, the compiler puts the tile products in accumulator registers and reads each
// one back)
template <typename T, int D>
__global__ __launch_bounds__(256, sizeof(T) == 2 && D == 64 ? 2 : 1) void chunk_bwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                        const T* __restrict__ V, const T* __restrict__ Klm,
                                                        const T* __restrict__ dO, const float* __restrict__ w,
                                                        const float* __restrict__ lse,
                                                        const int* __restrict__ chunk_off,
                                                        const int* __restrict__ pairs,
                                                        typename PartialOf<T>::type* __restrict__ dq_part,
                                                        float* __restrict__ Dpart,
                                                        typename PartialOf<T>::type* __restrict__ trash,
                                                        float* __restrict__ trash_f, float* __restrict__ dK,
                                                        float* __restrict__ dV, int L, int N, int k, float scale) {
  using S = BwdLds<T, D>;
  constexpr bool KV_IN_REGS = sizeof(T) == 2 && D == 64;
  int j, bh;
  xcd_map(j, bh);
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const int k1 = k + 1;
  __shared__ S s;
  {
    constexpr int EPP = 16 / Elem<T>::bytes, PER_ROW = D / EPP;
    const int64_t row0 = (int64_t)bh * L + (int64_t)j * 64;
    for (int p = tid; p < 64 * PER_ROW; p += 256) {
      const int key = p / PER_ROW, e0 = (p % PER_ROW) * EPP;
      const int4 kv = *reinterpret_cast<const int4*>(K + (row0 + key) * D + e0);
      const int4 vv = *reinterpret_cast<const int4*>(V + (row0 + key) * D + e0);
      *reinterpret_cast<int4*>(&s.k[key * S::KS + e0]) = kv;
      *reinterpret_cast<int4*>(&s.v[key * S::KS + e0]) = vv;
      T vals[EPP];
      __builtin_memcpy(vals, &kv, 16);
#pragma unroll
      for (int e = 0; e < EPP; ++e) s.kt[(e0 + e) * S::TS + key] = vals[e];
    }
  }
  __syncthreads();
  KVFrags<T, D, KV_IN_REGS> kv;
  kv.init(s);

  const int* co = chunk_off + (int64_t)bh * (N + 1);
  const int p_begin = co[j], p_end = co[j + 1];
  const int ntiles = 1 + (p_end - p_begin + 63) / 64;
  const int* pl = pairs + (int64_t)bh * L * k;
  const int64_t npl = (int64_t)L * k;
  const T* Qb = Q + (int64_t)bh * L * D;
  const T* Gb = dO + (int64_t)bh * L * D;
  const int qi = 16 * wv + r16;  // this lane's query slot in the tile

  f32x4_t accV[D / 16], accK[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    accV[db] = zero4();
    accK[db] = zero4();
  }
  // Software pipeline over the tiles (tile 0: the chunk's own queries, causal; tile i >= 1:
  // routed pairs 64(i-1) .. 64i-1) with two input sets used in turn: while a tile runs, the
  // query and upstream-gradient rows and the softmax statistics of the next tile load into
  // the other set, and the pair entries of the tile after it are read.  Every load is
  // unconditional (entries are read at clamped positions inside the list buffer, rows and
  // statistics at valid rows); lanes without a pair compute with p = 0 and store to scratch.
  struct TileIn {
    Frag<T> qf[D / 32], gf[D / 32];
    float lse, w;
    int t, slot;
    bool valid;
  };
  auto entry = [&](int tile) {
    const int64_t p = (int64_t)p_begin + (int64_t)(tile - 1) * 64 + qi;
    return pl[p < 0 ? 0 : (p < npl ? p : npl - 1)];
  };
  auto fetch = [&](int tile, int pe, TileIn& in) {
    if (tile == 0) {
      in.t = j * 64 + qi;
      in.slot = k;
      in.valid = true;
    } else {
      // list positions past the chunk's range may lie past the filled part of the list, whose
      // entries are undefined: lanes without a pair use their own-chunk row instead
      in.valid = p_begin + (tile - 1) * 64 + qi < p_end;
      in.t = in.valid ? (pe >> 5) : j * 64 + qi;
      in.slot = in.valid ? (pe & 31) : k;
    }
    const int64_t row = (int64_t)bh * L + in.t;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      in.qf[ks].load(Qb + (int64_t)in.t * D + ks * 32 + 8 * g);
      in.gf[ks].load(Gb + (int64_t)in.t * D + ks * 32 + 8 * g);
    }
    in.lse = lse[row * k1 + in.slot];
    in.w = w[row * k1 + in.slot];
  };
  auto process = [&](const TileIn& in, int tile) {
    const bool valid = in.valid;
    const int causal = tile == 0 ? qi : -1;
    const int64_t row = (int64_t)bh * L + in.t;
    const float lse_q = in.lse;
    const float w_q = valid ? in.w : 0.f;
    // S^T = K Q^T and dP^T = V dO^T: lane holds query qi, keys 16cb + 4g + i
    f32x4_t sc[4], dp[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      sc[cb] = zero4();
      dp[cb] = zero4();
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        mma(sc[cb], kv.k(s, cb, ks), in.qf[ks]);
        mma(dp[cb], kv.v(s, cb, ks), in.gf[ks]);
      }
    }
    // scale w_q p_i straight from the exponential: log2(scale w_q) joins the exponent's bias, so no
    // per-element multiply weights the probabilities.  Lanes without a pair (w_q = 0) and masked keys
    // give exp2(-inf) = 0; D_j = sum_i p_i dP_i comes back from the weighted sum with one reciprocal.
    // The staged w P and dA rows carry the factor scale: the dQ parts and dK need no further multiply,
    // and dV is divided by scale once, when it is written.
    const float c2 = scale * 1.44269504088896341f;  // scale * log2(e)
    const float sw = scale * w_q;
    const float bias = __log2f(sw) - lse_q * 1.44269504088896341f;
    const int lim = causal < 0 ? 63 : causal;
    float Dw = 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * cb + 4 * g + i;
        const float pw = __builtin_amdgcn_exp2f(key <= lim ? fmaf(sc[cb][i], c2, bias) : -INFINITY);
        sc[cb][i] = pw;
        Dw += pw * dp[cb][i];
      }
    Dw += lane_xor(Dw, 16);
    Dw += lane_xor(Dw, 32);
    const float Dj = sw > 0.f ? Dw * __builtin_amdgcn_rcpf(sw) : 0.f;
    // the four lane groups hold the same D_j
    *(valid ? Dpart + row * k1 + in.slot : trash_f) = Dj;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[cb][i] = sc[cb][i] * (dp[cb][i] - Dj);  // scale dA
    // dQ^T = K^T dA^T (key mapping of the B fragment as in the forward's P V)
    {
      Frag<T> daf[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = dp[2 * h + e / 4][e % 4];
        daf[h].set(v8);
      }
      typename PartialOf<T>::type* dst = valid ? dq_part + (row * k1 + in.slot) * D : trash;
      auto dq_block = [&](int db) {
        f32x4_t dq = zero4();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          Frag<T> a;
          const T* rowp = &s.kt[(16 * db + r16) * S::TS + 32 * h + 4 * g];
          a.load4x2(rowp, rowp + 16);
          mma(dq, a, daf[h]);
        }
        return dq;
      };
      // bf16 parts keep fp32's exponent range (no overflow whatever the scale of dQ); fp32 inputs keep fp32
      if constexpr (sizeof(typename PartialOf<T>::type) == 2) {
        // two 16-d blocks at a time: lane groups g and g ^ 1 swap one block's packed values, so that
        // each lane holds eight consecutive d and stores 16 bytes (even g: d 32p + 4g ..; odd g:
        // d 32p + 16 + 4(g - 1) ..), a row's 64 bytes per store instruction
        const bool odd = (g & 1) != 0;
#pragma unroll
        for (int p2 = 0; p2 < D / 32; ++p2) {
          const f32x4_t e = dq_block(2 * p2), o = dq_block(2 * p2 + 1);
          const uint32_t e0 = pack_bf16x2(e[0], e[1]), e1 = pack_bf16x2(e[2], e[3]);
          const uint32_t o0 = pack_bf16x2(o[0], o[1]), o1 = pack_bf16x2(o[2], o[3]);
          const uint32_t r0 = lane_xor_u32(odd ? e0 : o0, 16), r1 = lane_xor_u32(odd ? e1 : o1, 16);
          const uint4 v = odd ? make_uint4(r0, r1, o0, o1) : make_uint4(e0, e1, r0, r1);
          *reinterpret_cast<uint4*>(dst + 32 * p2 + (odd ? 16 + 4 * (g - 1) : 4 * g)) = v;
        }
      } else {
#pragma unroll
        for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4_t*>(dst + 16 * db + 4 * g) = dq_block(db);
      }
    }
    __syncthreads();  // previous tile's readers of the staged buffers are done
    // dO and w P (the dV operands); Q and dA (the dK operands)
    auto stage_v = [&]() {
      if constexpr (S::TR) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          *reinterpret_cast<bf16x8_t*>(&s.gt()[qi * S::QS + ks * 32 + 8 * g]) = in.gf[ks].v;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          u16x4_t pw;
#pragma unroll
          for (int i = 0; i < 4; ++i) pw[i] = f32_to_bf16(sc[cb][i]);
          *reinterpret_cast<u16x4_t*>(&s.pt[qi * S::TS + 16 * cb + 4 * g]) = pw;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) Elem<T>::store(s.gt(), (ks * 32 + 8 * g + e) * S::TS + qi, in.gf[ks].get(e));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) Elem<T>::store(s.pt, (16 * cb + 4 * g + i) * S::TS + qi, sc[cb][i]);
      }
    };
    auto stage_k = [&]() {
      if constexpr (S::TR) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          *reinterpret_cast<bf16x8_t*>(&s.qt[qi * S::QS + ks * 32 + 8 * g]) = in.qf[ks].v;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          u16x4_t da;
#pragma unroll
          for (int i = 0; i < 4; ++i) da[i] = f32_to_bf16(dp[cb][i]);
          *reinterpret_cast<u16x4_t*>(&s.dat()[qi * S::TS + 16 * cb + 4 * g]) = da;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) Elem<T>::store(s.qt, (ks * 32 + 8 * g + e) * S::TS + qi, in.qf[ks].get(e));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) Elem<T>::store(s.dat(), (16 * cb + 4 * g + i) * S::TS + qi, dp[cb][i]);
      }
    };
    // this wave's 16 keys: dV += (wP)^T dO, dK += dA^T Q (contraction over the 64 tile queries)
    auto products = [&](auto vc, auto kc) {
      constexpr bool DV = decltype(vc)::value != 0, DK = decltype(kc)::value != 0;
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        Frag<T> ap, ad;
        if constexpr (S::TR) {
          if constexpr (DV) ap.load_tr(s.pt, S::TS, kq * 32 + 8 * g, 16 * wv, lane);
          if constexpr (DK) ad.load_tr(s.dat(), S::TS, kq * 32 + 8 * g, 16 * wv, lane);
        } else {
          if constexpr (DV) ap.load(&s.pt[(16 * wv + r16) * S::TS + kq * 32 + 8 * g]);
          if constexpr (DK) ad.load(&s.dat()[(16 * wv + r16) * S::TS + kq * 32 + 8 * g]);
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          Frag<T> bg, bq;
          if constexpr (S::TR) {
            if constexpr (DV) bg.load_tr(s.gt(), S::QS, kq * 32 + 8 * g, 16 * db, lane);
            if constexpr (DK) bq.load_tr(s.qt, S::QS, kq * 32 + 8 * g, 16 * db, lane);
          } else {
            if constexpr (DV) bg.load(&s.gt()[(16 * db + r16) * S::TS + kq * 32 + 8 * g]);
            if constexpr (DK) bq.load(&s.qt[(16 * db + r16) * S::TS + kq * 32 + 8 * g]);
          }
          if constexpr (DV) mma(accV[db], ap, bg);
          if constexpr (DK) mma(accK[db], ad, bq);
        }
      }
    };
    if constexpr (S::SPLIT) {
      stage_v();
      __syncthreads();
      products(IntC<1>{}, IntC<0>{});
      __syncthreads();  // the dV operands are read: Q and dA take their buffers
      stage_k();
      __syncthreads();
      products(IntC<0>{}, IntC<1>{});
    } else {
      stage_v();
      stage_k();
      __syncthreads();
      products(IntC<1>{}, IntC<1>{});
    }
  };
  TileIn A, B;
  int e1 = entry(1);
  fetch(0, 0, A);
  for (int tile = 0;; tile += 2) {
    fetch(tile + 1, e1, B);
    const int e2 = entry(tile + 2);
    process(A, tile);
    if (tile + 1 >= ntiles) break;
    fetch(tile + 2, e2, A);
    e1 = entry(tile + 3);
    process(B, tile + 1);
    if (tile + 2 >= ntiles) break;
  }
  // write dK, dV of this chunk: lane holds d = 16db + r16, keys 16wv + 4g + i
  const int64_t krow0 = (int64_t)bh * L + (int64_t)j * 64 + 16 * wv + 4 * g;
  const float inv_scale = 1.f / scale;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dV[(krow0 + i) * D + 16 * db + r16] = accV[db][i] * inv_scale;
      dK[(krow0 + i) * D + 16 * db + r16] = accK[db][i];
    }
}

// Eight consecutive d of one query row per thread: D = sum_j w_j D_j, ds_j = w_j (D_j - D),
// dQ = sum_j (in-chunk part_j + scale ds_j Klm_j) in slot order.  K1M >= k + 1 slots are
// held in registers and every load of a row is issued before any is used (slots past k + 1
// and dropped slots read a valid address and are not used): two memory round trips per
// thread, the landmark rows once the indices are in.
// MM > 0: mlm <= MM landmarks per chunk (Klm [BH][N][mlm][D]).  A slot's score is the
// log-sum-exp of its landmark scores, so its term is scale ds_j sum_u p_u Klm_j,u with the shares
// p_u = softmax_u(scale qs . Klm_j,u) of the scoring query qs (Qs); these terms are summed in slot
// order apart from the in-chunk parts and added to them at the end.
// LF (landmark-free chunks): the own slot's landmark of query t is m_t, the causal mean of its chunk's
// keys up to t as the forward rounded it; the workgroup's rows lie in one chunk, whose means are
// staged in LDS from the keys Kf, and scale ds_own m_t is added after the slot sum.
template <typename T, int D, int K1M, bool RQ, int MM = 0, bool LF = false>
__global__ __launch_bounds__(256) void dq_reduce_kernel(const typename PartialOf<T>::type* __restrict__ dq_part,
                                                        const float* __restrict__ Dpart,
                                                        const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                        const T* __restrict__ Klm, float* __restrict__ ds_out,
                                                        float* __restrict__ dQ, float* __restrict__ dQr, int64_t rows,
                                                        int L, int N, int k, float scale, const T* __restrict__ Kf,
                                                        const T* __restrict__ Qs, int mlm) {
  constexpr int V8 = D / 8;                    // threads per row
  constexpr int LW = 2 * Elem<T>::bytes;       // 32-bit words of eight landmark elements
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / V8;
  const int c8 = (int)(gid % V8);
  float lmf[8];  // LF: this thread's eight elements of m_t
  if constexpr (LF) {
    // the launch covers whole chunks, so every thread of the workgroup reaches the barriers
    __shared__ float km[64 * (D + 1)];
    __shared__ float segsum[256 / D][D];
    const int64_t crow0 = ((int64_t)blockIdx.x * (256 / V8)) & ~(int64_t)63;
    stage_prefix_means<T, D>(Kf, crow0, km, segsum, threadIdx.x);
    const int qi = (int)(row - crow0);
#pragma unroll
    for (int e = 0; e < 8; ++e) lmf[e] = km[qi * (D + 1) + 8 * c8 + e];
  }
  if (row >= rows) return;
  const int k1 = k + 1;
  const int64_t bh = row / L;
  constexpr int VPP = (int)sizeof(typename PartialOf<T>::type) / 2;  // 16-byte loads per eight elements
  int jr[K1M];
  float wr[K1M], dr[K1M];
  uint4 raw[K1M][VPP];
#pragma unroll
  for (int r = 0; r < K1M; ++r) {
    const int64_t e = row * k1 + (r < k1 ? r : 0);
    jr[r] = idx[e];
    wr[r] = w[e];
    dr[r] = Dpart[e];
    const uint4* src = reinterpret_cast<const uint4*>(dq_part + e * D + 8 * c8);
#pragma unroll
    for (int h = 0; h < VPP; ++h) raw[r][h] = src[h];
  }
  bool ok[K1M];
  float Dsum = 0.f;
#pragma unroll
  for (int r = 0; r < K1M; ++r) {
    ok[r] = r < k1 && (r == k || (jr[r] >= 0 && jr[r] < N));
    if (ok[r]) Dsum += wr[r] * dr[r];
  }
  uint32_t lw[MM > 0 ? 1 : K1M][LW];
#pragma unroll
  for (int r = 0; r < (MM > 0 ? 0 : K1M); ++r) {
    const uint4* lp = reinterpret_cast<const uint4*>(Klm + (bh * N + (ok[r] ? jr[r] : 0)) * D + 8 * c8);
#pragma unroll
    for (int v = 0; v < LW / 4; ++v) {
      const uint4 x = lp[v];
      lw[r][4 * v] = x.x;
      lw[r][4 * v + 1] = x.y;
      lw[r][4 * v + 2] = x.z;
      lw[r][4 * v + 3] = x.w;
    }
  }
  // RQ: the landmark scores came from separate retrieval queries, whose gradient (the
  // ds * Klm terms) goes to dQr; dQ then keeps the in-chunk attention terms only.
  // LF: the own slot's landmark is not a K_lm row, its term is added after the sum;
  // several landmarks per chunk (MM > 0) add theirs below
  float acc[8], accr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = accr[e] = 0.f;
  float ds_own = 0.f;
#pragma unroll
  for (int r = 0; r < K1M; ++r) {
    if (!ok[r]) continue;
    const float ds = wr[r] * (dr[r] - Dsum);
    if (c8 == 0) ds_out[row * k1 + r] = ds;
    if (LF && r == k) ds_own = ds;
    const float sds = (MM > 0 || (LF && r == k)) ? 0.f : scale * ds;
    float h[8];
    if constexpr (VPP == 1) {
      const uint32_t wds[4] = {raw[r][0].x, raw[r][0].y, raw[r][0].z, raw[r][0].w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        h[2 * x] = __uint_as_float(wds[x] << 16);
        h[2 * x + 1] = __uint_as_float(wds[x] & 0xFFFF0000u);
      }
    } else {
      __builtin_memcpy(h, raw[r], 32);
    }
    if constexpr (MM > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += h[e];
    } else {
      T lm[8];
      __builtin_memcpy(lm, lw[r], 8 * sizeof(T));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (RQ) {
          acc[e] += h[e];
          accr[e] += sds * Elem<T>::to_f32(lm, e);
        } else {
          acc[e] += h[e] + sds * Elem<T>::to_f32(lm, e);
        }
      }
    }
  }
  if constexpr (MM > 0) {
    // the scoring query's eight elements, then SB slots at a time: their landmark rows are
    // requested together; unused slots read chunk 0's rows and add nothing (the same for every
    // lane of the row, so the shuffles stay within live rows)
    float qv[8];
    {
      T vals[8];
      constexpr int NQ = 8 * sizeof(T) / 16;
#pragma unroll
      for (int h = 0; h < NQ; ++h) {
        const int4 x = *reinterpret_cast<const int4*>(Qs + row * D + 8 * c8 + h * (8 / NQ));
        __builtin_memcpy(reinterpret_cast<char*>(vals) + 16 * h, &x, 16);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = Elem<T>::to_f32(vals, e);
    }
    float accm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) accm[e] = 0.f;
    constexpr int NV = Elem<T>::bytes == 2 ? 1 : 2;  // 16-byte loads per eight elements
    constexpr int SB = NV * MM <= 4 ? 4 : 2;
#pragma unroll
    for (int r0 = 0; r0 < K1M; r0 += SB) {
      if (r0 < k1) {
        int4 lraw[SB][MM][NV];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          const int r = r0 + sb < K1M ? r0 + sb : 0;
          const int j = (r0 + sb < K1M && ok[r]) ? jr[r] : 0;
#pragma unroll
          for (int u = 0; u < MM; ++u) {
            const T* lp = Klm + ((bh * N + j) * mlm + (u < mlm ? u : 0)) * D + 8 * c8;
#pragma unroll
            for (int h = 0; h < NV; ++h) lraw[sb][u][h] = *reinterpret_cast<const int4*>(lp + h * (8 / NV));
          }
        }
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          const int r = r0 + sb;
          if (r >= K1M || !ok[r]) continue;
          const float ds = wr[r] * (dr[r] - Dsum);
          float lv[MM][8], a[MM], amax = -INFINITY;
#pragma unroll
          for (int u = 0; u < MM; ++u) {
            T vals[8];
            __builtin_memcpy(vals, &lraw[sb][u][0], 8 * sizeof(T));
            float dot = 0.f;
            if (u < mlm) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                lv[u][e] = Elem<T>::to_f32(vals, e);
                dot += qv[e] * lv[u][e];
              }
            }
#pragma unroll
            for (int msk = 1; msk < V8; msk <<= 1) dot += lane_xor(dot, msk);
            a[u] = scale * dot;
            if (u < mlm) amax = fmaxf(amax, a[u]);
          }
          float z = 0.f;
#pragma unroll
          for (int u = 0; u < MM; ++u) z += u < mlm ? __expf(a[u] - amax) : 0.f;
          const float g = scale * ds / z;
#pragma unroll
          for (int u = 0; u < MM; ++u) {
            if (u >= mlm) continue;
            const float cu = g * __expf(a[u] - amax);
#pragma unroll
            for (int e = 0; e < 8; ++e) accm[e] += cu * lv[u][e];
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (RQ) accr[e] += accm[e];
      else acc[e] += accm[e];
    }
  }
  if constexpr (LF) {
    const float so = scale * ds_own;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (RQ) accr[e] += so * lmf[e];
      else acc[e] += so * lmf[e];
    }
  }
  float4* out = reinterpret_cast<float4*>(dQ + row * D + 8 * c8);
  out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if (RQ) {
    float4* outr = reinterpret_cast<float4*>(dQr + row * D + 8 * c8);
    outr[0] = make_float4(accr[0], accr[1], accr[2], accr[3]);
    outr[1] = make_float4(accr[4], accr[5], accr[6], accr[7]);
  }
}

// dKlm_j = scale * sum over the chunk's own tile and its routed pairs of ds_tj q_t.
// Tiles of 64 pairs; thread (pair p, quarter of d) accumulates across tiles; the 64 pair
// lanes are then summed in a fixed order.
template <typename T, int D>
__global__ __launch_bounds__(256) void klm_bwd_kernel(const T* __restrict__ Q, const float* __restrict__ ds,
                                                      const int* __restrict__ chunk_off, const int* __restrict__ pairs,
                                                      float* __restrict__ dKlm, int L, int N, int k, float scale,
                                                      int lf) {
  constexpr int QD = D / 4;                   // elements per thread
  constexpr int EPP = 16 / Elem<T>::bytes;    // elements per 16-byte load
  __shared__ float red[64][D + 1];
  int j, bh;
  xcd_map(j, bh);
  const int tid = threadIdx.x;
  const int p = tid >> 2, qt = tid & 3;
  const int k1 = k + 1;
  const int* co = chunk_off + (int64_t)bh * (N + 1);
  const int p_begin = co[j], p_end = co[j + 1];
  const int* pl = pairs + (int64_t)bh * L * k;
  const int ntiles = 1 + (p_end - p_begin + 63) / 64;
  float acc[QD];
#pragma unroll
  for (int e = 0; e < QD; ++e) acc[e] = 0.f;
  // tile 0 holds the chunk's own queries (their own slot), which do not score K_lm_j when chunks are
  // landmark-free.  TB tiles at a time: their pair entries are requested together, then their ds
  // values and query rows, so that a batch costs two memory round trips instead of two per tile;
  // the sums still run tile by tile in list order.  Lanes past the chunk's pairs read a valid row
  // (entries at clamped list positions, the chunk's first query) and add nothing.
  constexpr int TB = QD / EPP <= 2 ? 8 : 4;
  const int64_t npl = (int64_t)L * k;
  for (int tb = lf ? 1 : 0; tb < ntiles; tb += TB) {
    int pe[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int64_t pp = (int64_t)p_begin + (int64_t)(tb + u - 1) * 64 + p;
      pe[u] = pl[pp < 0 ? 0 : (pp < npl ? pp : npl - 1)];
    }
    bool ok[TB];
    float dsv[TB];
    int4 raw[TB][QD / EPP];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int tile = tb + u;
      int t, slot;
      if (tile == 0) {
        t = j * 64 + p;
        slot = k;
        ok[u] = true;
      } else {
        ok[u] = tile < ntiles && p_begin + (tile - 1) * 64 + p < p_end;
        t = ok[u] ? (pe[u] >> 5) : j * 64;
        slot = ok[u] ? (pe[u] & 31) : 0;
      }
      const int64_t row = (int64_t)bh * L + t;
      dsv[u] = ds[row * k1 + slot];
      const T* qp = Q + row * D + qt * QD;
#pragma unroll
      for (int v = 0; v < QD / EPP; ++v) raw[u][v] = *reinterpret_cast<const int4*>(qp + v * EPP);
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      if (!ok[u]) continue;
#pragma unroll
      for (int v = 0; v < QD / EPP; ++v) {
        T vals[EPP];
        __builtin_memcpy(vals, &raw[u][v], 16);
#pragma unroll
        for (int e = 0; e < EPP; ++e) acc[v * EPP + e] += dsv[u] * Elem<T>::to_f32(vals, e);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < QD; ++e) red[p][qt * QD + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float a = 0.f;
    for (int q = 0; q < 64; ++q) a += red[q][tid];
    dKlm[((int64_t)bh * N + j) * D + tid] = scale * a;
  }
}

template <typename T, int D>
static hipError_t bwd_t(const void* Q, const void* Qr, const void* K, const void* V, const void* Klm, bool lf, int mlm,
                        const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ, float* dQr,
                        float* dK, float* dV, float* dKlm, int BH, int L, int N, int k, float scale,
                        const BwdBufs& ws, hipStream_t st) {
  using PT = typename PartialOf<T>::type;
  const int64_t rows = (int64_t)BH * L;
  hipError_t e = launch_route(idx, ws.rb, BH, L, N, k, st);
  if (e != hipSuccess) return e;
  HILS_LAUNCH("chunk_bwd", (chunk_bwd_kernel<T, D>), dim3(N, BH), dim3(256), 0, st, (const T*)Q, (const T*)K,
              (const T*)V, (const T*)Klm, (const T*)dO, w, lse, ws.rb.chunk_off, ws.rb.pairs, (PT*)ws.dq_part, ws.Dpart,
              (PT*)ws.trash, ws.trash_f, dK, dV, L, N, k, scale);
  // rows * D / 8 threads: whole workgroups of whole chunks (L is a multiple of 64)
  const dim3 rgrid((unsigned)((rows * (D / 8) + 255) / 256));
  const bool rq = Qr != nullptr;
  const T* Qs = (const T*)(rq ? Qr : Q);
  auto reduce = [&](auto k1m, auto rqc, auto mmc, auto lfc) {
    constexpr int K1M = decltype(k1m)::value, MM = decltype(mmc)::value;
    constexpr bool RQ = decltype(rqc)::value != 0, LF = decltype(lfc)::value != 0;
    HILS_LAUNCH("dq_reduce", (dq_reduce_kernel<T, D, K1M, RQ, MM, LF>), rgrid, dim3(256), 0, st,
                (const PT*)ws.dq_part, ws.Dpart, idx, w, (const T*)Klm, ws.ds, dQ, dQr, rows, L, N, k, scale,
                (const T*)K, Qs, mlm);
  };
  auto reduce_m = [&](auto k1m, auto rqc) {
    if (lf) reduce(k1m, rqc, IntC<0>{}, IntC<1>{});
    else if (mlm == 0) reduce(k1m, rqc, IntC<0>{}, IntC<0>{});
    else if (mlm <= 2) reduce(k1m, rqc, IntC<2>{}, IntC<0>{});
    else reduce(k1m, rqc, IntC<4>{}, IntC<0>{});
  };
  if (k <= 8 && !rq) reduce_m(IntC<9>{}, IntC<0>{});
  else if (!rq) reduce_m(IntC<17>{}, IntC<0>{});
  else if (k <= 8) reduce_m(IntC<9>{}, IntC<1>{});
  else reduce_m(IntC<17>{}, IntC<1>{});
  // dKlm_j sums ds_tj times the query that scored the landmark
  if (mlm > 0) {
    // several landmarks per chunk: the score paths through every landmark's share
    hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    return launch_ml_bwd(Elem<T>::bytes == 2 ? 0 : 1, D, rq ? Qr : Q, Klm, mlm, ws.ds, ws.rb.chunk_off, ws.rb.pairs,
                         dKlm, BH, L, N, k, scale, st);
  }
  HILS_LAUNCH("klm_bwd", (klm_bwd_kernel<T, D>), dim3(N, BH), dim3(256), 0, st, (const T*)(rq ? Qr : Q), ws.ds,
              ws.rb.chunk_off, ws.rb.pairs, dKlm, L, N, k, scale, (int)lf);
  if (lf) {
    hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    return launch_lf_bwd(Elem<T>::bytes == 2 ? 0 : 1, D, rq ? Qr : Q, ws.ds, dKlm, dK, BH, L, N, k, scale, st);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(int dt, int d, const void* Q, const void* Qr, const void* K, const void* V, const void* Klm,
                      bool lf, int mlm, const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ,
                      float* dQr, float* dK, float* dV, float* dKlm, int BH, int L, int N, int k, float scale,
                      const BwdBufs& ws, hipStream_t st) {
  if ((Qr == nullptr) != (dQr == nullptr)) return hipErrorInvalidValue;
  if (dt == 0)
    return d == 64 ? bwd_t<bf16_t, 64>(Q, Qr, K, V, Klm, lf, mlm, dO, idx, w, lse, dQ, dQr, dK, dV, dKlm, BH, L, N, k,
                                       scale, ws, st)
                   : bwd_t<bf16_t, 128>(Q, Qr, K, V, Klm, lf, mlm, dO, idx, w, lse, dQ, dQr, dK, dV, dKlm, BH, L, N, k,
                                        scale, ws, st);
  return d == 64 ? bwd_t<float, 64>(Q, Qr, K, V, Klm, lf, mlm, dO, idx, w, lse, dQ, dQr, dK, dV, dKlm, BH, L, N, k,
                                   scale, ws, st)
                 : bwd_t<float, 128>(Q, Qr, K, V, Klm, lf, mlm, dO, idx, w, lse, dQ, dQr, dK, dV, dKlm, BH, L, N, k,
                                     scale, ws, st);
}

}  // namespace hils
