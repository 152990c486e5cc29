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
//            exclusive scan over chunks; also the chunk-major work items;
//   scatter  one wavefront per segment walks its pairs in (t, slot) order and
//            ranks equal chunks inside each 64-pair batch with ballots, so the
//            list of every chunk is sorted by (t, slot) on every run.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

constexpr int ROUTE_SEG_Q = 1024;  // queries per counting segment

int route_nseg(int L) { return (L + ROUTE_SEG_Q - 1) / ROUTE_SEG_Q; }
int route_max_items(int L, int N, int k, int ppi) {
  return N + (int)(((int64_t)L * k + ppi - 1) / ppi);
}

__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ idx, int* __restrict__ counts,
                                                          int L, int N, int k, int nseg) {
  extern __shared__ int hist[];
  const int seg = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  for (int j = tid; j < N; j += 256) hist[j] = 0;
  __syncthreads();
  const int t0 = seg * ROUTE_SEG_Q, t1 = min(L, t0 + ROUTE_SEG_Q);
  const int total = (t1 - t0) * k;
  for (int f = tid; f < total; f += 256) {
    const int t = t0 + f / k, r = f % k;
    const int j = idx[((int64_t)bh * L + t) * (k + 1) + r];
    if (j >= 0 && j < N) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  int* out = counts + ((int64_t)bh * nseg + seg) * N;
  for (int j = tid; j < N; j += 256) out[j] = hist[j];
}

// exclusive block scan of one int per thread (256 threads); returns the block total in *total
__device__ int block_excl_scan(int v, int* buf, int* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid];
  *total = buf[255];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(256) void route_scan_kernel(int* __restrict__ counts, int* __restrict__ chunk_off,
                                                         int2* __restrict__ items, int* __restrict__ n_items, int N,
                                                         int nseg, int ppi, int max_items) {
  __shared__ int buf[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  int carry_p = 0, carry_i = 0;
  for (int base = 0; base < N; base += 256) {
    const int j = base + tid;
    int tot = 0;
    if (j < N) {
      for (int s = 0; s < nseg; ++s) {
        int* p = counts + ((int64_t)bh * nseg + s) * N + j;
        const int cnum = *p;
        *p = tot;
        tot += cnum;
      }
    }
    const int nit = (tot + ppi - 1) / ppi;
    int sum_p, sum_i;
    const int ex_p = block_excl_scan(tot, buf, &sum_p);
    const int ex_i = block_excl_scan(nit, buf, &sum_i);
    if (j < N) {
      chunk_off[(int64_t)bh * (N + 1) + j] = carry_p + ex_p;
      int2* it = items + (int64_t)bh * max_items + carry_i + ex_i;
      for (int u = 0; u < nit; ++u) it[u] = make_int2(j, u);
    }
    carry_p += sum_p;
    carry_i += sum_i;
  }
  if (tid == 0) {
    chunk_off[(int64_t)bh * (N + 1) + N] = carry_p;
    n_items[bh] = carry_i;
  }
}

__global__ __launch_bounds__(64) void route_scatter_kernel(const int32_t* __restrict__ idx,
                                                           const int* __restrict__ segoff,
                                                           const int* __restrict__ chunk_off, int* __restrict__ pairs,
                                                           int L, int N, int k, int nseg, int nbits) {
  extern __shared__ int cur[];
  const int seg = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const int* so = segoff + ((int64_t)bh * nseg + seg) * N;
  const int* co = chunk_off + (int64_t)bh * (N + 1);
  for (int j = lane; j < N; j += 64) cur[j] = co[j] + so[j];
  __syncthreads();
  int* out = pairs + (int64_t)bh * L * k;
  const int t0 = seg * ROUTE_SEG_Q, t1 = min(L, t0 + ROUTE_SEG_Q);
  const int total = (t1 - t0) * k;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int base = 0; base < total; base += 64) {
    const int f = base + lane;
    int j = -1, t = 0, r = 0;
    if (f < total) {
      t = t0 + f / k;
      r = f % k;
      j = idx[((int64_t)bh * L + t) * (k + 1) + r];
    }
    const bool act = j >= 0 && j < N;
    uint64_t peers = __ballot(act);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = act && ((j >> b) & 1);
      const uint64_t ones = __ballot(bit);
      peers &= bit ? ones : ~ones;
    }
    int pos = 0;
    if (act) pos = cur[j] + __popcll(peers & below);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (act && (peers & below) == 0) cur[j] = pos + __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (act) out[pos] = (t << 5) | r;
  }
}

hipError_t launch_route(const int32_t* idx, const RouteBufs& rb, int BH, int L, int N, int k, hipStream_t st) {
  const size_t lds = (size_t)N * sizeof(int);
  hipLaunchKernelGGL(route_count_kernel, dim3(rb.nseg, BH), dim3(256), lds, st, idx, rb.counts, L, N, k, rb.nseg);
  hipLaunchKernelGGL(route_scan_kernel, dim3(BH), dim3(256), 0, st, rb.counts, rb.chunk_off, rb.items, rb.n_items, N,
                     rb.nseg, rb.pairs_per_item, rb.max_items);
  int nbits = 1;
  while ((1 << nbits) < N) ++nbits;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(rb.nseg, BH), dim3(64), lds, st, idx, rb.counts, rb.chunk_off,
                     rb.pairs, L, N, k, rb.nseg, nbits);
  return hipGetLastError();
}

}  // namespace hils
