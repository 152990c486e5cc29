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
// (D is taken from the forward's O, as flash-attention style backward passes do.)
//
// Kernels:
//   prep         D_t = dO_t . O_t per row.
//   chunk_bwd    one workgroup per chunk j: its own-chunk tile (the 64 queries
//                of chunk j, causal) and then the tiles of the queries that
//                selected j (routing lists, ascending (t, slot)).  dK_j, dV_j
//                and dKlm_j accumulate inside the workgroup in a fixed order,
//                so they are written once, without atomics, and bit-for-bit
//                reproducible.  Every pair writes its dQ contribution to a
//                per-(query, slot) buffer.
//   dq_reduce    dQ_t = sum over the query's slots, in slot order.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

template <typename T, int D> struct BwdLds {
  static constexpr int KS = D + (Elem<T>::bytes == 2 ? 8 : 4);   // rows indexed by key, d inside
  static constexpr int TS = 64 + (Elem<T>::bytes == 2 ? 8 : 4);  // rows of 64 (keys or tile queries)
  T k[64 * KS];
  T v[64 * KS];
  T kt[D * TS];   // K^T   [d][key]
  T qt[D * TS];   // Q^T   [d][tile query]
  T gt[D * TS];   // dO^T  [d][tile query]
  T pt[64 * TS];  // (w P)^T [key][tile query]
  T dat[64 * TS]; // dA^T  [key][tile query]
  float klm[D];
  float ds[64];
  float red[4][D];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                       float* __restrict__ Dt, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  float acc = 0.f;
  if (row < rows)
    for (int e = part * (D / 4); e < (part + 1) * (D / 4); ++e)
      acc += Elem<T>::to_f32(O, row * D + e) * Elem<T>::to_f32(dO, row * D + e);
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (row < rows && part == 0) Dt[row] = acc;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_bwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                        const T* __restrict__ V, const T* __restrict__ Klm,
                                                        const T* __restrict__ dO, const float* __restrict__ w,
                                                        const float* __restrict__ lse, const float* __restrict__ Dt,
                                                        const int* __restrict__ chunk_off,
                                                        const int* __restrict__ pairs, float* __restrict__ dq_part,
                                                        float* __restrict__ dK, float* __restrict__ dV,
                                                        float* __restrict__ dKlm, int L, int N, int k, float scale) {
  using S = BwdLds<T, D>;
  const int j = blockIdx.x, bh = blockIdx.y;
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
    for (int e = tid; e < D; e += 256) s.klm[e] = Elem<T>::to_f32(Klm, ((int64_t)bh * N + j) * D + e);
  }
  __syncthreads();

  const int* co = chunk_off + (int64_t)bh * (N + 1);
  const int p_begin = co[j], p_end = co[j + 1];
  const int ntiles = 1 + (p_end - p_begin + 63) / 64;
  const int* pl = pairs + (int64_t)bh * L * k;
  const T* Qb = Q + (int64_t)bh * L * D;
  const T* Gb = dO + (int64_t)bh * L * D;
  const int qi = 16 * wv + r16;  // this lane's query slot in the tile

  f32x4_t accV[D / 16], accK[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    accV[db] = zero4();
    accK[db] = zero4();
  }
  constexpr int PARTS = 256 / D;
  const int kd = tid % D, kpart = tid / D;
  float acc_klm = 0.f;

  for (int tile = 0; tile < ntiles; ++tile) {
    int t, slot, causal;
    bool valid;
    if (tile == 0) {
      t = j * 64 + qi;
      slot = k;
      causal = qi;
      valid = true;
    } else {
      const int p = p_begin + (tile - 1) * 64 + qi;
      valid = p < p_end;
      const int pe = valid ? pl[p] : 0;
      t = pe >> 5;
      slot = pe & 31;
      causal = -1;
    }
    const int64_t row = (int64_t)bh * L + t;
    Frag<T> qf[D / 32], gf[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      if (valid) {
        qf[ks].load(Qb + (int64_t)t * D + ks * 32 + 8 * g);
        gf[ks].load(Gb + (int64_t)t * D + ks * 32 + 8 * g);
      } else {
        qf[ks].zero();
        gf[ks].zero();
      }
    }
    const float lse_q = valid ? lse[row * k1 + slot] : 0.f;
    const float w_q = valid ? w[row * k1 + slot] : 0.f;
    const float D_q = valid ? Dt[row] : 0.f;
    // S^T = K Q^T and dP^T = V dO^T: lane holds query qi, keys 16cb + 4g + i
    f32x4_t sc[4], dp[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      sc[cb] = zero4();
      dp[cb] = zero4();
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        Frag<T> a, b;
        a.load(&s.k[(16 * cb + r16) * S::KS + ks * 32 + 8 * g]);
        b.load(&s.v[(16 * cb + r16) * S::KS + ks * 32 + 8 * g]);
        mma(sc[cb], a, qf[ks]);
        mma(dp[cb], b, gf[ks]);
      }
    }
    float Dj = 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * cb + 4 * g + i;
        const float p = (valid && (causal < 0 || key <= causal)) ? __expf(scale * sc[cb][i] - lse_q) : 0.f;
        sc[cb][i] = p;
        Dj += p * dp[cb][i];
      }
    Dj += __shfl_xor(Dj, 16);
    Dj += __shfl_xor(Dj, 32);
    const float ds_q = w_q * (Dj - D_q);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[cb][i] = w_q * sc[cb][i] * (dp[cb][i] - Dj);  // dA
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
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        f32x4_t dq = zero4();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          Frag<T> a;
          const T* rowp = &s.kt[(16 * db + r16) * S::TS + 32 * h + 4 * g];
          a.load4x2(rowp, rowp + 16);
          mma(dq, a, daf[h]);
        }
        if (valid) {
          float4 out;
          out.x = scale * (dq[0] + ds_q * s.klm[16 * db + 4 * g + 0]);
          out.y = scale * (dq[1] + ds_q * s.klm[16 * db + 4 * g + 1]);
          out.z = scale * (dq[2] + ds_q * s.klm[16 * db + 4 * g + 2]);
          out.w = scale * (dq[3] + ds_q * s.klm[16 * db + 4 * g + 3]);
          *reinterpret_cast<float4*>(dq_part + (row * k1 + slot) * D + 16 * db + 4 * g) = out;
        }
      }
    }
    __syncthreads();  // previous tile's readers of the transposed buffers are done
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        Elem<T>::store(s.qt, (ks * 32 + 8 * g + e) * S::TS + qi, qf[ks].get(e));
        Elem<T>::store(s.gt, (ks * 32 + 8 * g + e) * S::TS + qi, gf[ks].get(e));
      }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * cb + 4 * g + i;
        Elem<T>::store(s.pt, key * S::TS + qi, w_q * sc[cb][i]);
        Elem<T>::store(s.dat, key * S::TS + qi, dp[cb][i]);
      }
    if (g == 0) s.ds[qi] = ds_q;
    __syncthreads();
    // this wave's 16 keys: dV += (wP)^T dO, dK += dA^T Q (contraction over the 64 tile queries)
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      Frag<T> ap, ad;
      ap.load(&s.pt[(16 * wv + r16) * S::TS + kq * 32 + 8 * g]);
      ad.load(&s.dat[(16 * wv + r16) * S::TS + kq * 32 + 8 * g]);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        Frag<T> bg, bq;
        bg.load(&s.gt[(16 * db + r16) * S::TS + kq * 32 + 8 * g]);
        bq.load(&s.qt[(16 * db + r16) * S::TS + kq * 32 + 8 * g]);
        mma(accV[db], ap, bg);
        mma(accK[db], ad, bq);
      }
    }
    // dKlm_j += sum_q ds_q q  (thread: one d, a quarter or half of the queries)
    for (int q = kpart * (64 / PARTS); q < (kpart + 1) * (64 / PARTS); ++q)
      acc_klm += s.ds[q] * Elem<T>::to_f32(s.qt, kd * S::TS + q);
  }
  // write dK, dV of this chunk: lane holds d = 16db + r16, keys 16wv + 4g + i
  const int64_t krow0 = (int64_t)bh * L + (int64_t)j * 64 + 16 * wv + 4 * g;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dV[(krow0 + i) * D + 16 * db + r16] = accV[db][i];
      dK[(krow0 + i) * D + 16 * db + r16] = scale * accK[db][i];
    }
  s.red[kpart][kd] = acc_klm;
  __syncthreads();
  if (tid < D) {
    float a = 0.f;
    for (int p = 0; p < PARTS; ++p) a += s.red[p][tid];
    dKlm[((int64_t)bh * N + j) * D + tid] = scale * a;
  }
}

template <int D>
__global__ __launch_bounds__(256) void dq_reduce_kernel(const float* __restrict__ dq_part,
                                                        const int32_t* __restrict__ idx, float* __restrict__ dQ,
                                                        int64_t rows, int N, int k) {
  constexpr int V4 = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / V4;
  const int c4 = (int)(gid % V4);
  if (row >= rows) return;
  const int k1 = k + 1;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int r = 0; r < k1; ++r) {
    if (r < k && (idx[row * k1 + r] < 0 || idx[row * k1 + r] >= N)) continue;
    const float4 v = *reinterpret_cast<const float4*>(dq_part + (row * k1 + r) * D + 4 * c4);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>(dQ + row * D + 4 * c4) = acc;
}

template <typename T, int D>
static hipError_t bwd_t(const void* Q, const void* K, const void* V, const void* Klm, const void* O, const void* dO,
                        const int32_t* idx, const float* w, const float* lse, float* dQ, float* dK, float* dV,
                        float* dKlm, int BH, int L, int N, int k, float scale, const BwdBufs& ws, hipStream_t st) {
  const int64_t rows = (int64_t)BH * L;
  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, st, (const T*)O,
                     (const T*)dO, ws.Dt, rows);
  hipError_t e = launch_route(idx, ws.rb, BH, L, N, k, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_bwd_kernel<T, D>), dim3(N, BH), dim3(256), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                     (const T*)Klm, (const T*)dO, w, lse, ws.Dt, ws.rb.chunk_off, ws.rb.pairs, ws.dq_part, dK, dV,
                     dKlm, L, N, k, scale);
  hipLaunchKernelGGL((dq_reduce_kernel<D>), dim3((unsigned)((rows * (D / 4) + 255) / 256)), dim3(256), 0, st,
                     ws.dq_part, idx, dQ, rows, N, k);
  return hipGetLastError();
}

hipError_t launch_bwd(int dt, int d, const void* Q, const void* K, const void* V, const void* Klm, const void* O,
                      const void* dO, const int32_t* idx, const float* w, const float* lse, float* dQ, float* dK,
                      float* dV, float* dKlm, int BH, int L, int N, int k, float scale, const BwdBufs& ws,
                      hipStream_t st) {
  if (dt == 0)
    return d == 64 ? bwd_t<bf16_t, 64>(Q, K, V, Klm, O, dO, idx, w, lse, dQ, dK, dV, dKlm, BH, L, N, k, scale, ws, st)
                   : bwd_t<bf16_t, 128>(Q, K, V, Klm, O, dO, idx, w, lse, dQ, dK, dV, dKlm, BH, L, N, k, scale, ws,
                                        st);
  // fp32 inputs: head dim 64 only (the fp32 LDS tiles of d = 128 exceed a workgroup's LDS)
  if (d != 64) return hipErrorInvalidValue;
  return bwd_t<float, 64>(Q, K, V, Klm, O, dO, idx, w, lse, dQ, dK, dV, dKlm, BH, L, N, k, scale, ws, st);
}

}  // namespace hils
