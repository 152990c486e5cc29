// One decode step of HiLS attention: append, landmark scan, top-k, split-K
// chunk attention and fusion for a single new query per (b,h).
//
// Passages: "Hierarchical Sparse Attention Done Right" (ai-feeds summary),
// "Limitations" (at every decode step each chunk's landmark is scored, a cost
// linear in the context) and "Method" > "Key modules" items 1-3; the
// paper.oopus.info review, sections 3-4 (single-GPU bf16 decode at long
// context).  The operator is the prefill one for the query at position n:
// candidates are the completed chunks j < n/64, the open chunk n/64 is its own
// chunk (keys 64*(n/64) .. n).
//
// The step is bound by HBM reads of the landmark rows (every step reads all of
// them).  decode_scan streams them with 16-byte coalesced loads over many
// workgroups and writes one fp32 score per chunk (4 bytes per 128-256 bytes
// read).  decode_attend runs one 1024-thread workgroup per head.  One wavefront
// selects the top-m from the score row: the m-th largest of the 64 lane maxima
// (a wave-wide bitonic sort) bounds the m-th largest score from below, and the
// few scores at or above it are compacted with ballots and sorted exactly.  The
// k+1 kept chunks are then split over the 16 wavefronts (split-K), each reading
// its chunk's keys and values with 16-byte loads, and the weighted per-chunk
// outputs are fused in LDS in slot order.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

constexpr int DEC_ROWS = 256;   // landmark rows per scan workgroup
constexpr int DEC_GROUP = 32;   // chunks per group maximum written by the scan
constexpr int DEC_MAX_GROUPS = 16384 / DEC_GROUP;  // groups at the library's chunk limit

int decode_slices(int64_t n_ctx) { return (int)((n_ctx / 64 + DEC_ROWS - 1) / DEC_ROWS); }
// row strides of the per-head score row (a multiple of 32 floats) and group-maximum row
int64_t decode_score_stride(int64_t Nmax) { return (Nmax + 31) / 32 * 32; }
int64_t decode_gmax_stride(int64_t Nmax) { return (Nmax + DEC_ROWS - 1) / DEC_ROWS * (DEC_ROWS / DEC_GROUP); }

__device__ __forceinline__ int64_t decode_score_stride_d(int64_t Nmax) { return (Nmax + 31) / 32 * 32; }
__device__ __forceinline__ int64_t decode_gmax_stride_d(int64_t Nmax) {
  return (Nmax + DEC_ROWS - 1) / DEC_ROWS * (DEC_ROWS / DEC_GROUP);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_scan_kernel(const T* __restrict__ q, const T* __restrict__ k_new,
                                                          const T* __restrict__ v_new, T* __restrict__ Kc,
                                                          T* __restrict__ Vc, const T* __restrict__ Klm,
                                                          float* __restrict__ scores, float* __restrict__ gmax,
                                                          int64_t n, int64_t Lmax, int64_t Nmax, float scale) {
  constexpr int EPP = 16 / Elem<T>::bytes;  // elements per 16-byte piece
  constexpr int PIECES = D / EPP;           // pieces per row
  constexpr int RPR = 256 / PIECES;         // rows per round
  constexpr int ROUNDS = DEC_ROWS / RPR;
  const int s = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int c = (int)(n / 64);
  if (s == 0) {
    // append the new key and value (idempotent)
    for (int e = tid; e < D; e += 256) {
      Kc[((int64_t)bh * Lmax + n) * D + e] = k_new[(int64_t)bh * D + e];
      Vc[((int64_t)bh * Lmax + n) * D + e] = v_new[(int64_t)bh * D + e];
    }
  }
  const int j0 = s * DEC_ROWS;
  if (j0 >= c) return;
  const int piece = tid % PIECES, rr = tid / PIECES;
  float qv[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) qv[e] = Elem<T>::to_f32(q, (int64_t)bh * D + piece * EPP + e);
  const T* base = Klm + (int64_t)bh * Nmax * D + piece * EPP;
  int4 raw[ROUNDS];
#pragma unroll
  for (int round = 0; round < ROUNDS; ++round) {
    const int j = j0 + round * RPR + rr;
    raw[round] = j < c ? *reinterpret_cast<const int4*>(base + (int64_t)j * D) : make_int4(0, 0, 0, 0);
  }
  __shared__ float sc[DEC_ROWS];
  float* out = scores + (int64_t)bh * decode_score_stride_d(Nmax);
#pragma unroll
  for (int round = 0; round < ROUNDS; ++round) {
    T vals[EPP];
    __builtin_memcpy(vals, &raw[round], 16);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < EPP; ++e) dot += qv[e] * Elem<T>::to_f32(vals, e);
#pragma unroll
    for (int m = 1; m < PIECES; m <<= 1) dot += lane_xor(dot, m);
    const int j = j0 + round * RPR + rr;
    if (piece == 0) {
      const float v = j < c ? scale * dot : -INFINITY;
      sc[round * RPR + rr] = v;
      if (j < c) out[j] = v;
    }
  }
  __syncthreads();
  // maxima of the slice's groups of DEC_GROUP chunks (-inf past the last chunk)
  if (tid < DEC_ROWS / DEC_GROUP) {
    float mx = -INFINITY;
#pragma unroll 8
    for (int e = 0; e < DEC_GROUP; ++e) mx = fmaxf(mx, sc[tid * DEC_GROUP + e]);
    gmax[(int64_t)bh * decode_gmax_stride_d(Nmax) + s * (DEC_ROWS / DEC_GROUP) + tid] = mx;
  }
}

// Wave-wide bitonic sort, descending: afterwards lane i holds the i-th largest value.
template <typename K> __device__ __forceinline__ K wave_sort_desc(K v, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const K o = shfl_xor_any(v, stride);
      const bool desc = (lane & size) == 0;
      const bool lower = (lane & stride) == 0;
      const K hi = v > o ? v : o, lo = v > o ? o : v;
      v = (desc == lower) ? hi : lo;
    }
  }
  return v;
}

// top[0..m-1] = the m best keys of the score row sc[0..c) (score desc, index asc), given the
// maxima gm[] of its groups of DEC_GROUP chunks.  Run by one full wave.  Each lane holds
// the maxima of groups lane, lane+64, ...; the m-th largest lane maximum is a lower bound
// tau on the m-th best score (lane maxima are distinct candidates), so only groups whose
// maximum reaches tau are read, and their scores >= tau are sorted exactly.
__device__ void wave_select_topm(const float* __restrict__ sc, const float* __restrict__ gm, int c, int m,
                                 uint64_t* top, uint64_t* surv, int* cg, int lane) {
  constexpr int PER_LANE = 8;  // survivor slots per lane
  constexpr int MAXG = (16384 / DEC_GROUP + 63) / 64;  // group maxima per lane at the chunk limit
  const int ngroups = (c + DEC_GROUP - 1) / DEC_GROUP;
  // every load of the row issued before any is used: one memory round trip
  float gv[MAXG];
#pragma unroll
  for (int u = 0; u < MAXG; ++u) {
    const int gi = lane + 64 * u;
    gv[u] = gi < ngroups ? gm[gi] : -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < MAXG; ++u) mx = fmaxf(mx, gv[u]);
  const float sorted = wave_sort_desc(mx, lane);
  const float tau = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sorted), m - 1));
  // groups whose maximum reaches tau, compacted in LDS; then one pass of loads per 64 of them
  const uint64_t below = (1ull << lane) - 1ull;
  int ncand = 0;
#pragma unroll
  for (int u = 0; u < MAXG; ++u) {
    const int gi = lane + 64 * u;
    const bool is = gi < ngroups && gv[u] >= tau;
    const uint64_t mask = __ballot(is);
    if (is) cg[ncand + __popcll(mask & below)] = gi;
    ncand += __popcll(mask);
  }
  __builtin_amdgcn_wave_barrier();
  uint64_t mine[PER_LANE];
  int cnt = 0;
  bool ovf = false;
  for (int p0 = 0; p0 < ncand; p0 += 64) {
    const int gi = p0 + lane < ncand ? cg[p0 + lane] : -1;
    if (gi < 0) continue;
    const float4* gp = reinterpret_cast<const float4*>(sc + gi * DEC_GROUP);
    float4 v4[DEC_GROUP / 4];
#pragma unroll
    for (int u = 0; u < DEC_GROUP / 4; ++u) v4[u] = gp[u];
#pragma unroll
    for (int u = 0; u < DEC_GROUP / 4; ++u) {
      const float vv[4] = {v4[u].x, v4[u].y, v4[u].z, v4[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = gi * DEC_GROUP + 4 * u + e;
        if (j < c && vv[e] >= tau) {
#pragma unroll
          for (int q = 0; q < PER_LANE; ++q)
            if (q == cnt) mine[q] = make_key(vv[e], j);
          ovf |= cnt >= PER_LANE;
          ++cnt;
        }
      }
    }
  }
  // exclusive prefix of the per-lane counts
  int pre = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(pre, off);
    if (lane >= off) pre += o;
  }
  const int total = __builtin_amdgcn_readlane(pre, 63);
  pre -= cnt;
  const bool any_ovf = __ballot(ovf) != 0;
  if (!any_ovf && total <= 64) {
#pragma unroll
    for (int q = 0; q < PER_LANE; ++q)
      if (q < cnt) surv[pre + q] = mine[q];
    __builtin_amdgcn_wave_barrier();
    const uint64_t key = wave_sort_desc<uint64_t>(lane < total ? surv[lane] : (uint64_t)0, lane);
    if (lane < m) top[lane] = key;
  } else {
    // many exact ties at the bound: m passes of "largest key below the previous one"
    uint64_t prev = ~0ull;
    for (int r = 0; r < m; ++r) {
      uint64_t best = 0ull;
      for (int j = lane; j < c; j += 64) {
        const uint64_t key = make_key(sc[j], j);
        if (key < prev && key > best) best = key;
      }
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) {
        const uint64_t o = shfl_xor_u64(best, msk);
        best = o > best ? o : best;
      }
      if (lane == 0) top[r] = best;
      prev = best;
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// One 1024-thread workgroup per head: wave 0 selects, then each of the 16 wavefronts
// attends to one kept chunk (wave 0 also to a 17th), and the weighted per-chunk
// outputs are fused in LDS in slot order.  No cross-workgroup communication.
template <typename T, int D>
__global__ __launch_bounds__(1024) void decode_attend_kernel(const T* __restrict__ q, const T* __restrict__ Kc,
                                                             const T* __restrict__ Vc, const T* __restrict__ Klm,
                                                             const float* __restrict__ scores,
                                                             const float* __restrict__ gmax, T* __restrict__ o,
                                                             int32_t* __restrict__ idx, float* __restrict__ wout,
                                                             int64_t n, int64_t Lmax, int64_t Nmax, int k,
                                                             float scale) {
  constexpr int EPP = 16 / Elem<T>::bytes;
  constexpr int PIECES = D / EPP;   // 16-byte pieces per row (8 or 16 for bf16)
  constexpr int KPR = 64 / PIECES;  // keys per round when a row is spread over PIECES lanes
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = (int)(n / 64);
  const int m = min(k, c);
  __shared__ uint64_t top[16];
  __shared__ uint64_t surv[64];
  __shared__ int cgl[DEC_MAX_GROUPS];
  __shared__ float qs[D];
  __shared__ float sc_w[16][64];
  __shared__ float po[17][D];
  __shared__ float s_own_s;
  __shared__ float wsl[17];
  for (int e = tid; e < D; e += 1024) qs[e] = Elem<T>::to_f32(q, (int64_t)bh * D + e);
  if (wv == 0 && m > 0)
    wave_select_topm(scores + (int64_t)bh * decode_score_stride_d(Nmax), gmax + (int64_t)bh * decode_gmax_stride_d(Nmax),
                     c, m, top, surv, cgl, lane);
  __syncthreads();
  if (wv == 1) {
    float dot = 0.f;
    for (int e = lane; e < D; e += 64) dot += qs[e] * Elem<T>::to_f32(Klm, ((int64_t)bh * Nmax + c) * D + e);
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) dot += lane_xor(dot, msk);
    if (lane == 0) s_own_s = scale * dot;
  }
  __syncthreads();
  if (wv == 0) {
    // fusion weights of the kept slots (lane i < m: past slot i; lane 16: own chunk)
    const bool used = lane < m || lane == 16;
    const float sv = lane < m ? key_score(top[lane]) : (lane == 16 ? s_own_s : -INFINITY);
    float smax = sv;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) smax = fmaxf(smax, lane_xor(smax, msk));
    const float ev = used ? __expf(sv - smax) : 0.f;
    float den = ev;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) den += lane_xor(den, msk);
    if (lane < 17) wsl[lane] = ev / den;
  }
  __syncthreads();
  const int piece = lane % PIECES, kl = lane / PIECES;
  for (int item = wv; item <= m; item += 16) {
    const int r = item < m ? item : k;
    const int j = item < m ? key_index(top[item]) : c;
    const int nkeys = item < m ? 64 : (int)(n - (int64_t)c * 64) + 1;
    const int64_t row0 = (int64_t)bh * Lmax + (int64_t)j * 64;
    // keys and values of the chunk are requested together (one memory round trip) when a row
    // spans at most 8 lanes; wider rows load keys, then values, 8 rounds at a time.  A row is
    // spread over PIECES lanes, KPR rows per round.
    constexpr int UB = PIECES < 8 ? PIECES : 8;
    constexpr bool JOINT = PIECES <= 8;
    int4 vraw[JOINT ? PIECES : 1];
#pragma unroll
    for (int u0 = 0; u0 < PIECES; u0 += UB) {
      int4 kraw[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int key = (u0 + u) * KPR + kl;
        const bool ok = key < nkeys;
        kraw[u] = ok ? *reinterpret_cast<const int4*>(Kc + (row0 + key) * D + piece * EPP) : make_int4(0, 0, 0, 0);
        if constexpr (JOINT)
          vraw[u] = ok ? *reinterpret_cast<const int4*>(Vc + (row0 + key) * D + piece * EPP) : make_int4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        T vals[EPP];
        __builtin_memcpy(vals, &kraw[u], 16);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPP; ++e) dot += qs[piece * EPP + e] * Elem<T>::to_f32(vals, e);
#pragma unroll
        for (int msk = 1; msk < PIECES; msk <<= 1) dot += lane_xor(dot, msk);
        const int key = (u0 + u) * KPR + kl;
        if (piece == 0) sc_w[wv][key] = key < nkeys ? scale * dot : -INFINITY;
      }
    }
    __builtin_amdgcn_wave_barrier();
    const float v = sc_w[wv][lane];
    float mx = v;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) mx = fmaxf(mx, lane_xor(mx, msk));
    const float p = __expf(v - mx);
    float sum = p;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) sum += lane_xor(sum, msk);
    __builtin_amdgcn_wave_barrier();
    sc_w[wv][lane] = p;
    __builtin_amdgcn_wave_barrier();
    float acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u0 = 0; u0 < PIECES; u0 += UB) {
      int4 raw[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        if constexpr (JOINT) {
          raw[u] = vraw[u0 + u];
        } else {
          const int key = (u0 + u) * KPR + kl;
          raw[u] = key < nkeys ? *reinterpret_cast<const int4*>(Vc + (row0 + key) * D + piece * EPP)
                               : make_int4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        T vals[EPP];
        __builtin_memcpy(vals, &raw[u], 16);
        const float pk = sc_w[wv][(u0 + u) * KPR + kl];
#pragma unroll
        for (int e = 0; e < EPP; ++e) acc[e] += pk * Elem<T>::to_f32(vals, e);
      }
    }
#pragma unroll
    for (int msk = PIECES; msk < 64; msk <<= 1)
#pragma unroll
      for (int e = 0; e < EPP; ++e) acc[e] += lane_xor(acc[e], msk);
    const int slot = item < m ? item : 16;
    const float f = wsl[slot] / sum;
    if (kl == 0) {
#pragma unroll
      for (int e = 0; e < EPP; ++e) po[slot][piece * EPP + e] = f * acc[e];
    }
    (void)r;
  }
  __syncthreads();
  for (int e = tid; e < D; e += 1024) {
    float acc = 0.f;
    for (int i = 0; i < m; ++i) acc += po[i][e];
    acc += po[16][e];
    Elem<T>::store(o, (int64_t)bh * D + e, acc);
  }
  if (tid <= k) {
    const bool used = tid < m || tid == k;
    idx[(int64_t)bh * (k + 1) + tid] = tid == k ? c : (used ? key_index(top[tid]) : -1);
    wout[(int64_t)bh * (k + 1) + tid] = tid == k ? wsl[16] : (used ? wsl[tid] : 0.f);
  }
}

template <typename T, int D>
static hipError_t decode_t(const void* q, const void* k_new, const void* v_new, void* Kc, void* Vc, const void* Klm,
                           int64_t n, int64_t Lmax, int64_t Nmax, void* o, int32_t* idx, float* w, int BH, int k,
                           float scale, const DecodeBufs& ws, hipStream_t st) {
  const int S = decode_slices(n);
  HILS_LAUNCH("decode_scan", (decode_scan_kernel<T, D>), dim3(S > 0 ? S : 1, BH), dim3(256), 0, st, (const T*)q,
              (const T*)k_new, (const T*)v_new, (T*)Kc, (T*)Vc, (const T*)Klm, ws.scores, ws.gmax, n, Lmax, Nmax, scale);
  HILS_LAUNCH("decode_attend", (decode_attend_kernel<T, D>), dim3(BH), dim3(1024), 0, st, (const T*)q, (const T*)Kc,
              (const T*)Vc, (const T*)Klm, ws.scores, ws.gmax, (T*)o, idx, w, n, Lmax, Nmax, k, scale);
  return hipGetLastError();
}

hipError_t launch_decode(int dt, int d, const void* q, const void* k_new, const void* v_new, void* Kc, void* Vc,
                         const void* Klm, int64_t n, int64_t Lmax, int64_t Nmax, void* o, int32_t* idx, float* w,
                         int BH, int k, float scale, const DecodeBufs& ws, hipStream_t st) {
  if (dt == 0)
    return d == 64 ? decode_t<bf16_t, 64>(q, k_new, v_new, Kc, Vc, Klm, n, Lmax, Nmax, o, idx, w, BH, k, scale, ws, st)
                   : decode_t<bf16_t, 128>(q, k_new, v_new, Kc, Vc, Klm, n, Lmax, Nmax, o, idx, w, BH, k, scale, ws,
                                           st);
  return d == 64 ? decode_t<float, 64>(q, k_new, v_new, Kc, Vc, Klm, n, Lmax, Nmax, o, idx, w, BH, k, scale, ws, st)
                 : decode_t<float, 128>(q, k_new, v_new, Kc, Vc, Klm, n, Lmax, Nmax, o, idx, w, BH, k, scale, ws, st);
}

}  // namespace hils
