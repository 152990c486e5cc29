// Causal key means of landmark-free chunks, shared by the landmark-free kernels and the backward's
// dQ reduction (which adds the own slot's term against the same rounded means the forward used).
#pragma once
#include "hils_device.h"

namespace hils {

// The chunk's keys (rows row0 .. row0+63) staged as fp32 in km (row stride D + 1), then replaced by
// their causal means: row r becomes the mean of rows 0..r, rounded to the element type like a
// landmark row.  The prefix sums run as 256/D row segments at once, offset by the earlier segments.
// Ends with a barrier.
template <typename T, int D>
__device__ __forceinline__ void stage_prefix_means(const T* __restrict__ K, int64_t row0, float* km,
                                                   float (*segsum)[D], int tid) {
  constexpr int EPP = 16 / Elem<T>::bytes;
  constexpr int PIECES = D / EPP;
  constexpr int RPR = 256 / PIECES;
  constexpr int KS = D + 1;
  constexpr int SEG = 256 / D;
  constexpr int RS = 64 / SEG;
  {
    const int piece = tid % PIECES, rr = tid / PIECES;
#pragma unroll
    for (int r0 = 0; r0 < 64; r0 += RPR) {
      const int r = r0 + rr;
      const int4 raw = *reinterpret_cast<const int4*>(K + (row0 + r) * D + piece * EPP);
      T vals[EPP];
      __builtin_memcpy(vals, &raw, 16);
#pragma unroll
      for (int e = 0; e < EPP; ++e) km[r * KS + piece * EPP + e] = Elem<T>::to_f32(vals, e);
    }
  }
  __syncthreads();
  const int e = tid % D, sg = tid / D;
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < RS; ++i) {
    const int r = sg * RS + i;
    run += km[r * KS + e];
    km[r * KS + e] = run;
  }
  segsum[sg][e] = run;
  __syncthreads();
  float off = 0.f;
  for (int j = 0; j < sg; ++j) off += segsum[j][e];
#pragma unroll
  for (int i = 0; i < RS; ++i) {
    const int r = sg * RS + i;
    T m[1];
    Elem<T>::store(m, 0, (km[r * KS + e] + off) / (float)(r + 1));
    km[r * KS + e] = Elem<T>::to_f32(m, 0);
  }
  __syncthreads();
}

}  // namespace hils
