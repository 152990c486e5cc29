// Routing inversion: from each query's selected chunks to each chunk's queries.
//
// The pages attribute HiLS's speed to reading only the retrieved chunks' keys
// and values ("Hierarchical Sparse Attention Done Right", ai-feeds summary,
// "Method" > "Key modules" item 3; abstract: sparse KV access and
// computation).  With independent queries the chunks chosen by neighbouring
// queries rarely coincide, so the kernels here regroup the (query, slot) pairs
// by chunk: every chunk's keys and values are then read once and its queries
// form full MFMA tiles.
//
// A deterministic counting sort per (b,h):
//   count    per segment of queries, an LDS histogram over chunks;
//   scan     per chunk, exclusive offsets over segments and a global
//            exclusive scan over chunks; also the chunk-major work items
//            (for short sequences folded into the scatter workgroups);
//   scatter  one wavefront per segment walks its pairs in (t, slot) order and
//            ranks equal chunks inside each 64-pair batch with ballots, so the
//            list of every chunk is sorted by (t, slot) on every run; it also
//            records where each pair went (the inverse map, written in query
//            order), so per-pair results stored in list order can be gathered
//            back per query.
#include <atomic>

#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

// queries per counting segment: short sequences use short segments (more parallel
// scatter wavefronts), long ones longer segments (fewer per-segment counters)
int route_seg_q(int L) { return L / 64 <= 1024 ? 256 : 1024; }
int route_nseg(int L) { return (L + route_seg_q(L) - 1) / route_seg_q(L); }
int route_max_items(int L, int N, int k, int ppi) {
  return N + (int)(((int64_t)L * k + ppi - 1) / ppi);
}

// Pair f of a run of queries is (query f / k, slot f % k).  The quotient comes from a float
// product: for f < 2^15 and k <= 32, (f + 1/2) / k lies at least 1/(2k) from an integer while the
// product's rounding error stays below 2^-8, so truncation gives f / k exactly (a run holds at most
// 1024 queries x 16 slots).
__device__ __forceinline__ int2 pair_of(int f, int k, float rk) {
  const int q = (int)(((float)f + 0.5f) * rk);
  return make_int2(q, f - __mul24(q, k));
}

__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ idx, int* __restrict__ counts,
                                                          int L, int N, int k, int nseg, int seg_q) {
  extern __shared__ int hist[];
  const int seg = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  for (int j = tid; j < N; j += 256) hist[j] = 0;
  __syncthreads();
  const int t0 = seg * seg_q, t1 = min(L, t0 + seg_q);
  const int total = (t1 - t0) * k;
  const int32_t* idx_s = idx + ((int64_t)bh * L + t0) * (k + 1);
  const float rk = 1.f / (float)k;
  for (int f0 = 0; f0 < total; f0 += 8 * 256) {
    int jj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int f = f0 + u * 256 + tid;
      const int2 qr = pair_of(f, k, rk);
      jj[u] = f < total ? idx_s[qr.x * (k + 1) + qr.y] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (jj[u] >= 0 && jj[u] < N) atomicAdd(&hist[jj[u]], 1);
  }
  __syncthreads();
  int* out = counts + ((int64_t)bh * nseg + seg) * N;
  for (int j = tid; j < N; j += 256) out[j] = hist[j];
}

// exclusive block scan of one int per thread (NW wavefronts); returns the block total in *total.
// Each wavefront scans its 64 values, then adds the totals of the wavefronts before it.
template <int NW = 4> __device__ int block_excl_scan(int v, int* buf, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) buf[wv] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int tw = buf[w];
    before += w < wv ? tw : 0;
    all += tw;
  }
  *total = all;
  __syncthreads();  // buf is reused by the next call
  return before + incl - v;
}

// One 1024-thread workgroup per (b,h): a thread per chunk forms that chunk's per-segment offsets
// (its column of the counts, read 32 segments at a time), then block scans give the chunk offsets
// and the work items; long sequences take N / 1024 such rounds.
constexpr int ROUTE_SCAN_T = 1024;
__global__ __launch_bounds__(ROUTE_SCAN_T) void route_scan_kernel(int* __restrict__ counts, int* __restrict__ chunk_off,
                                                                  int4* __restrict__ items, int* __restrict__ n_items,
                                                                  int N, int nseg, int ppi, int max_items) {
  __shared__ int buf[ROUTE_SCAN_T / 64];
  const int bh = blockIdx.x, tid = threadIdx.x;
  int carry_p = 0, carry_i = 0;
  for (int base = 0; base < N; base += ROUTE_SCAN_T) {
    const int j = base + tid;
    int tot = 0;
    if (j < N) {
      for (int s0 = 0; s0 < nseg; s0 += 32) {
        int cv[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) cv[u] = s0 + u < nseg ? counts[((int64_t)bh * nseg + s0 + u) * N + j] : 0;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          if (s0 + u < nseg) counts[((int64_t)bh * nseg + s0 + u) * N + j] = tot;
          tot += cv[u];
        }
      }
    }
    const int nit = (tot + ppi - 1) / ppi;
    int sum_p, sum_i;
    const int ex_p = block_excl_scan<ROUTE_SCAN_T / 64>(tot, buf, &sum_p);
    const int ex_i = block_excl_scan<ROUTE_SCAN_T / 64>(nit, buf, &sum_i);
    if (j < N) {
      const int off = carry_p + ex_p;
      chunk_off[(int64_t)bh * (N + 1) + j] = off;
      int4* it = items + (int64_t)bh * max_items + carry_i + ex_i;
      for (int u = 0; u < nit; ++u) it[u] = make_int4(j, off + u * ppi, min(off + tot, off + (u + 1) * ppi), 0);
    }
    carry_p += sum_p;
    carry_i += sum_i;
  }
  if (tid == 0) {
    chunk_off[(int64_t)bh * (N + 1) + N] = carry_p;
    n_items[bh] = carry_i;
  }
}

// NW wavefronts per segment: wave w takes the w-th share of the segment's queries.  Each
// wave first counts its pairs per chunk (LDS histogram); the cursors of wave w then start
// after the pairs of waves 0..w-1 in every chunk, so the list keeps the (t, slot) order.
//
// FUSED (short sequences, N <= 256 chunks and at most 64 segments): there is no scan pass;
// every segment's workgroup reads the head's raw counts itself (thread j: chunk j), forms
// its segment offsets and, with a block scan, the chunk offsets, and the first segment's
// workgroup also writes the chunk offsets and the work items.
constexpr int ROUTE_FUSED_MAX_N = 256, ROUTE_FUSED_MAX_SEG = 64;

template <int NW, bool FUSED>
__global__ __launch_bounds__(64 * NW) void route_scatter_kernel(const int32_t* __restrict__ idx,
                                                                const int* __restrict__ segoff,
                                                                int* __restrict__ chunk_off,
                                                                int4* __restrict__ items, int* __restrict__ n_items,
                                                                int* __restrict__ pairs, int* __restrict__ pos_of,
                                                                int L, int N, int k, int nseg, int nbits, int seg_q,
                                                                int ppi, int max_items) {
  extern __shared__ int cur_all[];  // [NW][N]
  int seg, bh;
  xcd_map(seg, bh);  // a head's segments run in order on one XCD: its list writes merge in one L2
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int* so = segoff + ((int64_t)bh * nseg + seg) * N;
  const int* co = chunk_off + (int64_t)bh * (N + 1);
  __shared__ int so_s[FUSED ? ROUTE_FUSED_MAX_N : 1], co_s[FUSED ? ROUTE_FUSED_MAX_N : 1];
  const int t0 = seg * seg_q, t1 = min(L, t0 + seg_q);
  const int qpw = (seg_q + NW - 1) / NW;
  const int tw0 = min(t1, t0 + wv * qpw), tw1 = min(t1, tw0 + qpw);
  const int total = (tw1 - tw0) * k;
  const int32_t* idx_w = idx + ((int64_t)bh * L + tw0) * (k + 1);
  // short sequences: the wave's chunk ids (at most 256 queries x 16 slots per segment) are read
  // once, for the histogram and the ranking, and requested before the counts so that the two
  // memory round trips overlap
  constexpr int UBF = FUSED ? 256 * 16 / (NW * 64) : 1;
  int jr[UBF];
  const float rk = 1.f / (float)k;
  if constexpr (FUSED) {
#pragma unroll
    for (int u = 0; u < UBF; ++u) {
      const int f = u * 64 + lane;
      const int2 qr = pair_of(f, k, rk);
      jr[u] = f < total ? idx_w[qr.x * (k + 1) + qr.y] : -1;
    }
  }
  if constexpr (FUSED) {
    static_assert(64 * NW >= ROUTE_FUSED_MAX_N, "one thread per chunk");
    __shared__ int buf[NW];
    const int j = tid;
    int before = 0, tot = 0;
    {
      // segment rows past nseg are skipped as a whole (a uniform branch); lanes past the chunks
      // read a valid column and count nothing
      const int* so_h = segoff + (int64_t)bh * nseg * N + min(j, N - 1);
      int cv[ROUTE_FUSED_MAX_SEG];
#pragma unroll
      for (int u = 0; u < ROUTE_FUSED_MAX_SEG; ++u) cv[u] = u < nseg ? so_h[u * N] : 0;
#pragma unroll
      for (int u = 0; u < ROUTE_FUSED_MAX_SEG; ++u) {
        if (u < seg) before += cv[u];
        if (u < nseg) tot += cv[u];
      }
      if (j >= N) before = tot = 0;
    }
    int all, sum_i;
    const int off = block_excl_scan<NW>(tot, buf, &all);
    const int nit = j < N ? (tot + ppi - 1) / ppi : 0;
    const int ex_i = block_excl_scan<NW>(nit, buf, &sum_i);
    if (j < N) {
      so_s[j] = before;
      co_s[j] = off;
      if (seg == 0) {
        chunk_off[(int64_t)bh * (N + 1) + j] = off;
        int4* it = items + (int64_t)bh * max_items + ex_i;
        for (int u = 0; u < nit; ++u) it[u] = make_int4(j, off + u * ppi, min(off + tot, off + (u + 1) * ppi), 0);
      }
    }
    if (seg == 0 && tid == 0) {
      chunk_off[(int64_t)bh * (N + 1) + N] = all;
      n_items[bh] = sum_i;
    }
    __syncthreads();
  }
  auto seg_off = [&](int j) { if constexpr (FUSED) return so_s[j]; else return so[j]; };
  auto chunk_start = [&](int j) { if constexpr (FUSED) return co_s[j]; else return co[j]; };
  int* cur = cur_all + wv * N;
  if constexpr (NW > 1) {
    for (int i = tid; i < NW * N; i += 64 * NW) cur_all[i] = 0;
    __syncthreads();
    if constexpr (FUSED) {
#pragma unroll
      for (int u = 0; u < UBF; ++u)
        if (jr[u] >= 0 && jr[u] < N) atomicAdd(&cur[jr[u]], 1);
    } else {
      for (int f0 = 0; f0 < total; f0 += 8 * 64) {
        int jj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int f = f0 + u * 64 + lane;
          const int2 qr = pair_of(f, k, rk);
          jj[u] = f < total ? idx_w[qr.x * (k + 1) + qr.y] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (jj[u] >= 0 && jj[u] < N) atomicAdd(&cur[jj[u]], 1);
      }
    }
    __syncthreads();
    for (int j = tid; j < N; j += 64 * NW) {
      int run = chunk_start(j) + seg_off(j);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int h = cur_all[w * N + j];
        cur_all[w * N + j] = run;
        run += h;
      }
    }
  } else {
    for (int j = lane; j < N; j += 64) cur[j] = chunk_start(j) + seg_off(j);
  }
  __syncthreads();
  int* out = pairs + (int64_t)bh * L * k;
  int* pos_w = pos_of ? pos_of + ((int64_t)bh * L + tw0) * k : nullptr;
  const uint64_t below = (1ull << lane) - 1ull;
  // one 64-pair batch: rank equal chunks by lane (ballots over the chunk bits), take the slots
  auto place = [&](int f, int j) {
    const bool act = j >= 0 && j < N;
    uint64_t peers = __ballot(act);
    if (peers == 0) {
      if (pos_w && f < total) pos_w[f] = -1;
      return;
    }
    for (int b = 0; b < nbits; ++b) {
      const bool bit = act && ((j >> b) & 1);
      const uint64_t ones = __ballot(bit);
      peers &= bit ? ones : ~ones;
    }
    int pos = 0;
    if (act) pos = cur[j] + __popcll(peers & below);
    // LDS instructions of one wavefront execute in order: every lane's read of cur[j]
    // precedes the leader's update below
    __builtin_amdgcn_wave_barrier();
    if (act && (peers & below) == 0) cur[j] = pos + __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (act) {
      const int2 qr = pair_of(f, k, rk);
      out[pos] = ((tw0 + qr.x) << 5) | qr.y;
    }
    if (pos_w && f < total) pos_w[f] = act ? pos : -1;
  };
  if constexpr (FUSED) {
#pragma unroll
    for (int u = 0; u < UBF; ++u) {
      if (u * 64 >= total) break;
      place(u * 64 + lane, jr[u]);
    }
  } else {
    constexpr int U = 8;  // batches whose chunk ids are loaded together
    for (int b0 = 0; b0 < total; b0 += U * 64) {
      int jj[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int f = b0 + u * 64 + lane;
        const int2 qr = pair_of(f, k, rk);
        jj[u] = f < total ? idx_w[qr.x * (k + 1) + qr.y] : -1;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) place(b0 + u * 64 + lane, jj[u]);
    }
  }
}

// Long sequences (many chunks): the pairs of one segment reach every chunk's list in runs of a
// few entries, and 4-byte stores scattered over the head's whole list (larger than an L2)
// would each cost a partial memory write.  This variant ranks the pairs exactly as above but
// stages the segment's part of every list in LDS, in list order, then copies it out: the runs
// of consecutive entries of one list are stored together by neighbouring lanes.
// LDS (16-bit where the values are local positions below seg_q * k <= 16384):
//   cur[NW][N]  per-wave histogram, then per-wave cursors (local positions)
//   lbase[N+1]  start of each chunk's run in the staged segment
//   delta[N]    list position minus local position, per chunk
//   stage[seg_q * k]  (local query << 5) | slot, in list order
//   tag[N]      lane of the last store per chunk (8-bit): finds batches without repeated chunks
constexpr int ROUTE_STAGED_MAX_N = 2048;
constexpr int ROUTE_STAGED_NW = 8;
inline size_t route_staged_lds(int N, int seg_q, int k, int nw) {
  auto al = [](size_t b) { return (b + 15) & ~(size_t)15; };
  return al((size_t)nw * N * 2) + al((size_t)(N + 1) * 2) + al((size_t)N * 4) + al((size_t)seg_q * k * 2) +
         al((size_t)N);
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void route_scatter_staged_kernel(const int32_t* __restrict__ idx,
                                                                       const int* __restrict__ segoff,
                                                                       const int* __restrict__ chunk_off,
                                                                       int* __restrict__ pairs,
                                                                       int* __restrict__ pos_of, int L, int N, int k,
                                                                       int nseg, int nbits, int seg_q) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  auto al = [](size_t b) { return (b + 15) & ~(size_t)15; };
  uint16_t* cur_all = reinterpret_cast<uint16_t*>(lds_raw);
  uint16_t* lbase = reinterpret_cast<uint16_t*>(lds_raw + al((size_t)NW * N * 2));
  int* delta = reinterpret_cast<int*>(lds_raw + al((size_t)NW * N * 2) + al((size_t)(N + 1) * 2));
  uint16_t* stage = reinterpret_cast<uint16_t*>(lds_raw + al((size_t)NW * N * 2) + al((size_t)(N + 1) * 2) +
                                                al((size_t)N * 4));
  uint8_t* tag = reinterpret_cast<uint8_t*>(lds_raw + al((size_t)NW * N * 2) + al((size_t)(N + 1) * 2) +
                                            al((size_t)N * 4) + al((size_t)seg_q * k * 2));
  int seg, bh;
  xcd_map(seg, bh);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int* so = segoff + ((int64_t)bh * nseg + seg) * N;
  const int* co = chunk_off + (int64_t)bh * (N + 1);
  const int t0 = seg * seg_q, t1 = min(L, t0 + seg_q);
  const int qpw = (seg_q + NW - 1) / NW;
  const int tw0 = min(t1, t0 + wv * qpw), tw1 = min(t1, tw0 + qpw);
  const int total = (tw1 - tw0) * k;
  const int32_t* idx_w = idx + ((int64_t)bh * L + tw0) * (k + 1);
  // the wave's chunk ids, all requested at once and kept for the ranking pass
  constexpr int UB = 1024 * 16 / (NW * 64);  // batches of 64 pairs a wave holds at most
  int jr[UB];
  const float rk = 1.f / (float)k;
#pragma unroll
  for (int u = 0; u < UB; ++u) {
    const int f = u * 64 + lane;
    const int2 qr = pair_of(f, k, rk);
    jr[u] = f < total ? idx_w[qr.x * (k + 1) + qr.y] : -1;
  }
  uint32_t* cur_words = reinterpret_cast<uint32_t*>(cur_all);
  for (int i = tid; i < (NW * N + 1) / 2; i += 64 * NW) cur_words[i] = 0u;
  __syncthreads();
  // per-wave histograms (16-bit counters, added as halves of 32-bit words)
  uint16_t* cur = cur_all + wv * N;
#pragma unroll
  for (int u = 0; u < UB; ++u)
    if (jr[u] >= 0 && jr[u] < N) {
      const int e = wv * N + jr[u];
      atomicAdd(&cur_words[e >> 1], 1u << (16 * (e & 1)));
    }
  __syncthreads();
  // the segment's run of every chunk: exclusive scan of the chunk totals (CPT chunks a
  // thread), then the per-wave cursors inside each run
  {
    constexpr int CPT = ROUTE_STAGED_MAX_N / (64 * NW);
    int tot[CPT];
    int sum = 0;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = tid * CPT + u;
      int t = 0;
      if (j < N) {
#pragma unroll
        for (int w = 0; w < NW; ++w) t += cur_all[w * N + j];
      }
      tot[u] = t;
      sum += t;
    }
    __shared__ int buf[NW];
    int all;
    int run = block_excl_scan<NW>(sum, buf, &all);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = tid * CPT + u;
      if (j < N) {
        lbase[j] = (uint16_t)run;
        delta[j] = co[j] + so[j] - run;
        int r = run;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int h = cur_all[w * N + j];
          cur_all[w * N + j] = (uint16_t)r;
          r += h;
        }
      }
      run += tot[u];
    }
    if (tid == 0) lbase[N] = (uint16_t)all;
  }
  __syncthreads();
  int* pos_w = pos_of ? pos_of + ((int64_t)bh * L + tw0) * k : nullptr;
  const uint64_t below = (1ull << lane) - 1ull;
  {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (u * 64 >= total) break;
      const int f = u * 64 + lane;
      const int j = jr[u];
      const bool act = j >= 0 && j < N;
      uint64_t peers = __ballot(act);
      if (peers == 0) {
        if (pos_w && f < total) pos_w[f] = -1;
        continue;
      }
      // Most batches name every chunk once.  Each lane stores its number in its chunk's tag
      // and reads it back: lanes of this wave that share a chunk read one value in the same
      // instruction, so at least one of them sees another lane's number (another wave's
      // store can only add false alarms).  Without a repeat every lane takes one slot.
      if (act) tag[j] = (uint8_t)lane;
      __builtin_amdgcn_wave_barrier();
      const bool repeat = __any(act && tag[j] != lane);
      int lpos = 0;
      if (!repeat) {
        if (act) {
          lpos = cur[j];
          cur[j] = (uint16_t)(lpos + 1);
        }
      } else {
        for (int b = 0; b < nbits; ++b) {
          const bool bit = act && ((j >> b) & 1);
          const uint64_t ones = __ballot(bit);
          peers &= bit ? ones : ~ones;
        }
        if (act) lpos = cur[j] + __popcll(peers & below);
        // LDS instructions of one wavefront execute in order: every lane's read of cur[j]
        // precedes the leader's update below
        __builtin_amdgcn_wave_barrier();
        if (act && (peers & below) == 0) cur[j] = (uint16_t)(lpos + __popcll(peers));
      }
      __builtin_amdgcn_wave_barrier();
      if (act) {
        const int2 qr = pair_of(f, k, rk);
        stage[lpos] = (uint16_t)(((tw0 - t0 + qr.x) << 5) | qr.y);
      }
      if (pos_w && f < total) pos_w[f] = act ? lpos + delta[j] : -1;
    }
  }
  __syncthreads();
  // copy-out, eight lanes per chunk: each chunk's run goes to its list as one piece
  int* out = pairs + (int64_t)bh * L * k;
  const int sub = lane & 7;
  for (int j = wv * 8 + (lane >> 3); j < N; j += NW * 8) {
    const int p0 = lbase[j], p1 = lbase[j + 1], dj = delta[j];
    for (int p = p0 + sub; p < p1; p += 8) {
      const int v = stage[p];
      out[p + dj] = ((t0 + (v >> 5)) << 5) | (v & 31);
    }
  }
}

hipError_t launch_route(const int32_t* idx, const RouteBufs& rb, int BH, int L, int N, int k, hipStream_t st) {
  const size_t lds = (size_t)N * sizeof(int);
  HILS_LAUNCH("route_count", route_count_kernel, dim3(rb.nseg, BH), dim3(256), lds, st, idx, rb.counts, L, N, k, rb.nseg,
              rb.seg_q);
  int nbits = 1;
  while ((1 << nbits) < N) ++nbits;
  if (N <= ROUTE_FUSED_MAX_N && rb.nseg <= ROUTE_FUSED_MAX_SEG && rb.seg_q <= 256) {
    // eight wavefronts per segment (shorter ranking chains) while the grid is one round of
    // workgroups; four when there are many segments
    if ((int64_t)rb.nseg * BH <= 512)
      HILS_LAUNCH("route_scatter", (route_scatter_kernel<8, true>), dim3(rb.nseg, BH), dim3(512), 8 * lds, st, idx,
                  rb.counts, rb.chunk_off, rb.items, rb.n_items, rb.pairs, rb.pos_of, L, N, k, rb.nseg, nbits,
                  rb.seg_q, rb.pairs_per_item, rb.max_items);
    else
      HILS_LAUNCH("route_scatter", (route_scatter_kernel<4, true>), dim3(rb.nseg, BH), dim3(256), 4 * lds, st, idx,
                  rb.counts, rb.chunk_off, rb.items, rb.n_items, rb.pairs, rb.pos_of, L, N, k, rb.nseg, nbits,
                  rb.seg_q, rb.pairs_per_item, rb.max_items);
    return hipGetLastError();
  }
  HILS_LAUNCH("route_scan", route_scan_kernel, dim3(BH), dim3(ROUTE_SCAN_T), 0, st, rb.counts, rb.chunk_off, rb.items, rb.n_items, N,
                     rb.nseg, rb.pairs_per_item, rb.max_items);
  if (N <= ROUTE_STAGED_MAX_N && rb.seg_q * k <= 16384) {
    // more than 64 KiB of dynamic LDS per workgroup is opted into once per device
    static std::atomic<uint64_t> lds_set{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
    if (!bit || !(lds_set.load() & bit)) {
      e = hipFuncSetAttribute((const void*)route_scatter_staged_kernel<ROUTE_STAGED_NW>,
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)route_staged_lds(ROUTE_STAGED_MAX_N, 1024, 16, ROUTE_STAGED_NW));
      if (e != hipSuccess) return e;
      lds_set.fetch_or(bit);
    }
    HILS_LAUNCH("route_scatter", route_scatter_staged_kernel<ROUTE_STAGED_NW>, dim3(rb.nseg, BH),
                dim3(64 * ROUTE_STAGED_NW), route_staged_lds(N, rb.seg_q, k, ROUTE_STAGED_NW), st, idx, rb.counts,
                rb.chunk_off, rb.pairs, rb.pos_of, L, N, k, rb.nseg, nbits, rb.seg_q);
    return hipGetLastError();
  }
  // longer sequences: one wavefront per segment
  HILS_LAUNCH("route_scatter", (route_scatter_kernel<1, false>), dim3(rb.nseg, BH), dim3(64), lds, st, idx,
              rb.counts, rb.chunk_off, rb.items, rb.n_items, rb.pairs, rb.pos_of, L, N, k, rb.nseg, nbits, rb.seg_q,
              rb.pairs_per_item, rb.max_items);
  return hipGetLastError();
}

}  // namespace hils
