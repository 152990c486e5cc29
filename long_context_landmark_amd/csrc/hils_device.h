// Device-side building blocks shared by the HiLS kernels (gfx950 / CDNA4).
//
// Operand fragments follow the 16x16x32 bf16 MFMA lane layout of gfx950:
// lane l feeds row (A) / column (B) l%16 and the eight consecutive k-elements
// 8*(l/16) .. 8*(l/16)+7 of a 32-wide k block; the 4 accumulator values of
// lane l are rows 4*(l/16)+i, column l%16.  An fp32 fragment holds the same
// eight k-elements and is consumed by eight 16x16x4 fp32 MFMAs, so callers see
// one layout for both element types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct bf16_t {  // storage type of a bf16 element
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even: gfx950 converts in hardware (v_cvt_pk_bf16_f32,
// two values per instruction)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int bytes = 2;
  __device__ static float to_f32(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  __device__ static void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static constexpr int bytes = 4;
  __device__ static float to_f32(const float* p, int64_t i) { return p[i]; }
  __device__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};

// Storage type of per-pair intermediate rows (chunk outputs, in-chunk dQ parts): bf16 bits for 16-bit
// inputs, fp32 for fp32 inputs (their intermediates keep the inputs' precision).
template <typename T> struct PartialOf { using type = uint16_t; };
template <> struct PartialOf<float> { using type = float; };

// Eight consecutive k-elements of one row, as one MFMA operand fragment.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  bf16x8_t v;
  __device__ __forceinline__ void zero() {
    u16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
    v = __builtin_bit_cast(bf16x8_t, z);
  }
  // 16-byte aligned load of 8 consecutive elements
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const bf16x8_t*>(p); }
  // elements e=0..3 from p0, e=4..7 from p1 (each 8-byte aligned)
  __device__ __forceinline__ void load4x2(const bf16_t* p0, const bf16_t* p1) {
    u16x4_t a = *reinterpret_cast<const u16x4_t*>(p0);
    u16x4_t b = *reinterpret_cast<const u16x4_t*>(p1);
    u16x8_t c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    v = __builtin_bit_cast(bf16x8_t, c);
  }
  __device__ __forceinline__ void set(const float (&f)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)f[e];
  }
  __device__ __forceinline__ float get(int e) const {
    u16x8_t c = __builtin_bit_cast(u16x8_t, v);
    return bf16_to_f32(c[e]);
  }
  // Fragment of the transpose of a row-major LDS matrix X (row stride `stride` elements, a
  // multiple of 4; c0 a multiple of 4): lane l receives X[r0 + e][c0 + l % 16] for e = 0..7, where
  // r0 differs per group of 16 lanes.  Uses the transposing LDS read: in each 16-lane group, lane
  // i receives element i % 4 of the 8-byte pieces addressed by lanes 4e + i / 4 (e = 0..3) of the
  // group, so lane s addresses row r0 + s / 4, columns c0 + 4 (s % 4) .. + 3 (checked on the device
  // with an in-bounds probe).
  __device__ __forceinline__ void load_tr(const bf16_t* X, int stride, int r0, int c0, int lane) {
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    const int s = lane & 15;
    const bf16_t* p = X + (r0 + (s >> 2)) * stride + c0 + 4 * (s & 3);
    const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
    const i16x4_t b =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p + 4 * stride));
    const u16x8_t c = {(uint16_t)a[0], (uint16_t)a[1], (uint16_t)a[2], (uint16_t)a[3],
                       (uint16_t)b[0], (uint16_t)b[1], (uint16_t)b[2], (uint16_t)b[3]};
    v = __builtin_bit_cast(bf16x8_t, c);
  }
};
template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  __device__ __forceinline__ void load(const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void load4x2(const float* p0, const float* p1) {
    float4 a = *reinterpret_cast<const float4*>(p0);
    float4 b = *reinterpret_cast<const float4*>(p1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void set(const float (&f)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f[e];
  }
  __device__ __forceinline__ float get(int e) const { return v[e]; }
};

// Gathered rows as MFMA fragments.  A fragment holds row r16 = lane & 15 in every lane, so
// loading it directly has each quad of neighbouring lanes read four different rows, which
// the vector memory path serves at a quarter of its rate.  Instead lane 4a + b loads the
// 16 bytes at elements 8b.. of each 32-element step of row a (a quad reads 64 consecutive
// bytes), and the fragment is then assembled across lanes: lane (r16, g) takes the value
// of lane 4 r16 + g, which holds the same elements of the same row.
__device__ __forceinline__ int quad_row(int lane) { return lane >> 2; }
__device__ __forceinline__ int quad_piece(int lane) { return lane & 3; }
__device__ __forceinline__ void frag_from_quads(Frag<bf16_t>& f, int lane) {
  const int src = (4 * (lane & 15) + (lane >> 4)) * 4;  // byte address of the source lane
  u32x4_t u = __builtin_bit_cast(u32x4_t, f.v);
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)u[e]);
  f.v = __builtin_bit_cast(bf16x8_t, u);
}

// acc += A(16x32) * B(32x16) for one k block
__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() {
  f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// ---------------------------------------------------------------------------
// Selection keys: a 64-bit integer whose unsigned order is the selection order
// (higher fp32 score first, lower chunk index on equal scores).
__device__ __forceinline__ uint32_t ordered_bits(float s) {
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_float(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t make_key(float s, int32_t j) {
  s = s + 0.0f;  // -0 and +0 compare equal as scores; give them one key
  return ((uint64_t)ordered_bits(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}
__device__ __forceinline__ int32_t key_index(uint64_t key) { return (int32_t)(0xFFFFFFFFu - (uint32_t)key); }
__device__ __forceinline__ float key_score(uint64_t key) { return unordered_float((uint32_t)(key >> 32)); }

// A compile-time integer passed as a value (selects an unrolled variant of a generic lambda).
template <int N> struct IntC {
  static constexpr int value = N;
};

template <typename K> __device__ __forceinline__ void cmpswap_desc(K& a, K& b) {
  K hi = a > b ? a : b;
  K lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// Sort 16 values descending in registers (bitonic network, fully unrolled).
template <typename K> __device__ __forceinline__ void sort16_desc(K (&a)[16]) {
#pragma unroll
  for (int size = 2; size <= 16; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        int p = i ^ stride;
        if (p > i) {
          bool desc = (i & size) == 0;
          if (desc) cmpswap_desc(a[i], a[p]);
          else cmpswap_desc(a[p], a[i]);
        }
      }
    }
  }
}

// Sort the first 8 of N values descending: the 19-comparator network of depth 6 (optimal
// for 8 inputs; checked on all 0/1 inputs).
template <typename K, int N> __device__ __forceinline__ void sort8_desc(K (&a)[N]) {
  static_assert(N >= 8, "needs 8 values");
  constexpr int net[19][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}, {0, 4}, {1, 5}, {2, 6}, {3, 7}, {0, 1}, {2, 3},
                              {4, 5}, {6, 7}, {2, 4}, {3, 5}, {1, 4}, {3, 6}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
  for (int c = 0; c < 19; ++c) cmpswap_desc(a[net[c][0]], a[net[c][1]]);
}

// The first 8 values are bitonic; sort them descending.
template <typename K, int N> __device__ __forceinline__ void bitonic_merge8_desc(K (&a)[N]) {
#pragma unroll
  for (int stride = 4; stride > 0; stride >>= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int p = i ^ stride;
      if (p > i) cmpswap_desc(a[i], a[p]);
    }
  }
}

// The 8 largest of 16 values, sorted descending, into a[0..7] (a[8..15] are left unordered).
template <typename K> __device__ __forceinline__ void top8_of16_desc(K (&a)[16]) {
  K b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = a[8 + i];
  sort8_desc(a);
  sort8_desc(b);
  // a[i] vs b[7-i]: the larger halves form a bitonic sequence holding the top 8
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = a[i] > b[7 - i] ? a[i] : b[7 - i];
  bitonic_merge8_desc(a);
}

// a is bitonic; sort it descending.
template <typename K> __device__ __forceinline__ void bitonic_merge16_desc(K (&a)[16]) {
#pragma unroll
  for (int stride = 8; stride > 0; stride >>= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int p = i ^ stride;
      if (p > i) cmpswap_desc(a[i], a[p]);
    }
  }
}

// Value of lane (l ^ mask) for the lane-xor patterns of butterfly reductions and
// bitonic networks, without the LDS crossbar (ds_bpermute) that __shfl_xor uses:
//   mask 1, 2: DPP quad permutations [1,0,3,2] and [2,3,0,1];
//   mask 4:    row_half_mirror (l -> 7-l in each 8) then quad permutation [3,2,1,0];
//   mask 8:    DPP row rotate by 8 inside each row of 16;
//   mask 16:   v_permlane16_swap (exchanges the odd rows of one copy with the even
//              rows of the other: element 0 holds row r^1 on odd rows, element 1 on even);
//   mask 32:   v_permlane32_swap (the same between the two halves of the wave).
// Other masks fall back to __shfl_xor.  After loop unrolling the mask is a constant
// and the switch folds away.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, int mask) {
  const int iv = (int)v;
  switch (mask) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);
    case 4: {
      const int h = __builtin_amdgcn_mov_dpp(iv, 0x141, 0xF, 0xF, true);
      return (uint32_t)__builtin_amdgcn_mov_dpp(h, 0x1B, 0xF, 0xF, true);
    }
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, true);
    case 16: {
      const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (__lane_id() & 16) ? sw[0] : sw[1];
    }
    case 32: {
      const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (__lane_id() & 32) ? sw[0] : sw[1];
    }
    default: return (uint32_t)__shfl_xor(iv, mask);
  }
}
__device__ __forceinline__ float lane_xor(float v, int mask) {
  return __uint_as_float(lane_xor_u32(__float_as_uint(v), mask));
}
__device__ __forceinline__ int lane_xor(int v, int mask) { return (int)lane_xor_u32((uint32_t)v, mask); }
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = lane_xor_u32((uint32_t)v, mask), hi = lane_xor_u32((uint32_t)(v >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return lane_xor(v, mask); }
__device__ __forceinline__ uint64_t shfl_xor_any(uint64_t v, int m) { return shfl_xor_u64(v, m); }
__device__ __forceinline__ float shfl_xor_any(float v, int m) { return shfl_xor_f(v, m); }
__device__ __forceinline__ uint32_t shfl_xor_any(uint32_t v, int m) { return lane_xor_u32(v, m); }

// Wave-wide bitonic sort, descending: afterwards lane i holds the i-th largest value.
// Each stage keeps, per lane, the partner's value when it is larger and this lane
// keeps the maximum of the pair, or smaller and it keeps the minimum.  With W < 64 every
// group of W consecutive lanes is sorted on its own (lane W g + i holds its i-th largest).
template <typename K, int W = 64> __device__ __forceinline__ K wave_sort_desc(K v, int lane) {
#pragma unroll
  for (int size = 2; size <= W; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const K o = shfl_xor_any(v, stride);
      const bool keep_max = ((lane & size) == 0) == ((lane & stride) == 0);
      v = ((o > v) == keep_max) ? o : v;
    }
  }
  return v;
}

// Butterfly reductions over all 64 lanes (every lane receives the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += lane_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, lane_xor(v, m));
  return v;
}

// Lanes l and l^mask each hold a descending list of 16; afterwards both hold the
// 16 largest of the union, descending.
template <typename K> __device__ __forceinline__ void merge16_with_lane(K (&a)[16], int mask) {
  K b[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) b[i] = shfl_xor_any(a[i], mask);
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = a[i] > b[15 - i] ? a[i] : b[15 - i];
  bitonic_merge16_desc(a);
}

// The first 8 values of this lane and of lane (l ^ mask), both sorted descending: keep the 8
// largest of the 16, sorted descending, in a[0..7].
template <typename K, int N> __device__ __forceinline__ void merge8_with_lane(K (&a)[N], int mask) {
  K b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = shfl_xor_any(a[i], mask);
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = a[i] > b[7 - i] ? a[i] : b[7 - i];
  bitonic_merge8_desc(a);
}

__device__ __forceinline__ float wave_max_xor(float v, int from_mask, int to_mask) {
#pragma unroll
  for (int m = from_mask; m <= to_mask; m <<= 1) v = fmaxf(v, lane_xor(v, m));
  return v;
}

// XCD-aware grid mapping for a 2D grid (x = work index inside a head, y = head).
// Workgroups are dispatched to the 8 XCDs in round-robin order of their linear
// id, each XCD with its own L2.  When the head count is a multiple of 8, remap so
// that all workgroups of a head run on one XCD, in x order: the head's data then
// stays in one L2 instead of eight.  Otherwise the plain mapping is kept.
constexpr int NUM_XCD = 8;
constexpr int64_t L2_BYTES_PER_XCD = 4 << 20;
constexpr int64_t MALL_BYTES = (int64_t)256 << 20;  // memory-side (Infinity) cache
__device__ __forceinline__ void xcd_map(int& x, int& y) {
  const int gx = (int)gridDim.x, gy = (int)gridDim.y;
  x = (int)blockIdx.x;
  y = (int)blockIdx.y;
  if (gy % NUM_XCD) return;
  const int64_t lin = (int64_t)blockIdx.y * gx + blockIdx.x;
  const int xcd = (int)(lin % NUM_XCD);
  const int64_t r = lin / NUM_XCD;
  y = (int)(r / gx) * NUM_XCD + xcd;
  x = (int)(r % gx);
}

}  // namespace hils
