// Shared device helpers for the gfx950 kernels (wave64, bf16 MFMA).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace park {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even float -> bfloat16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// A 32-bit word as a pair of bfloat16. Takes the word by value: bit-casting an element of a vector
// register in place has been seen to read the wrong element, so callers pass a scalar copy.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// Two floats to packed bfloat16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 32x32x16 bf16 MFMA. Lane l: A row l%32, B column l%32, each with k = (l/32)*8 .. +7;
// D element i of lane l is row (i/4)*8 + (l/32)*4 + i%4, column l%32.
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA. Lane l: A row l%16, B column l%16, each with k = (l/16)*8 .. +7;
// D element i of lane l is row (l/16)*4 + i, column l%16.
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Eight consecutive elements of a row as packed bf16 (fp32 data is rounded to bf16).
template <typename T>
__device__ __forceinline__ u32x4_t load8_bf16(const T* p);

template <>
__device__ __forceinline__ u32x4_t load8_bf16<uint16_t>(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

template <>
__device__ __forceinline__ u32x4_t load8_bf16<float>(const float* p) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
  u32x4_t r;
  r[0] = pack_bf16x2(a[0], a[1]);
  r[1] = pack_bf16x2(a[2], a[3]);
  r[2] = pack_bf16x2(b[0], b[1]);
  r[3] = pack_bf16x2(b[2], b[3]);
  return r;
}

// Eight consecutive elements as fp32 (16- or 32-byte aligned pointer).
__device__ __forceinline__ void load8_f32(const uint16_t* p, float* out) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    out[2 * q] = __uint_as_float(v[q] << 16);
    out[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8_f32(const float* p, float* out) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    out[q] = a[q];
    out[4 + q] = b[q];
  }
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float load_f32<float>(const float* p, int64_t i) {
  return p[i];
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, kWave);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Inclusive prefix sum over a wave in lane order (fixed order, deterministic).
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    T u = __shfl_up(v, o, kWave);
    if (l >= o) v += u;
  }
  return v;
}

// Block-wide exclusive scan of one value per thread (blockDim.x a multiple of 64, <= 1024).
// `scratch` holds >= 17 T. Returns the exclusive prefix; *total receives the block total.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* scratch, T* total) {
  const int l = lane_id();
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  T inc = wave_inclusive_scan(v);
  if (l == kWave - 1) scratch[w] = inc;
  __syncthreads();
  if (w == 0) {
    T s = (l < nw) ? scratch[l] : T(0);
    T si = wave_inclusive_scan(s);
    if (l < nw) scratch[l] = si - s;
    if (l == nw - 1) scratch[16] = si;
  }
  __syncthreads();
  T res = scratch[w] + inc - v;
  *total = scratch[16];
  __syncthreads();
  return res;
}

// First output of a SplitMix64 generator seeded with `seed` (Steele, Lea & Flood, OOPSLA 2014: the
// state advances by the golden-ratio increment and passes through a 64-bit finaliser). The counter
// streams of the seeding and of the block sampling both draw from it.
__device__ __forceinline__ uint64_t splitmix_first(uint64_t seed) {
  uint64_t z = seed + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
#define PARK_LDS __attribute__((address_space(3)))

// Chunk swizzle of LDS row r. Two read patterns must be bank-conflict free:
//  - K (ds_read_b128): a 16-lane group reads one logical chunk of rows {0-3, 16-19, 4-7, 20-23}
//    (or the same set + 8), so those 16 rows need distinct swizzles (and, for 8-lane phases,
//    distinct low 3 bits within {0-3, 16-19} and within {4-7, 20-23});
//  - V (ds_read_b64_tr_b16): a half-wave reads an aligned group of four chunks from four
//    consecutive rows 4a..4a+3 (a quarter-wave: two chunks), so bits 2-3 (and bits 1-2) of the
//    swizzle must differ across those four rows.
// D = 128 (16 chunks per row): sw = 2 (g ^ 2g) ^ ((r >> 2) & 1) * 2 ^ ((r >> 4) & 1), g = r & 3,
// i.e. {0, 6, 12, 10} by r & 3 with the bit-0/bit-1 flips separating the row quartets.
// D = 64 (8 chunks, two rows per 256-byte bank sweep): rows of equal parity in a K group need
// distinct swizzles, rows r and r + 2 of a V quartet need different bit 2.
template <int CPR>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (CPR == 16) {
    const int g = r & 3;
    return (2 * (g ^ (g << 1))) ^ (((r >> 2) & 1) << 1) ^ ((r >> 4) & 1);
  } else {
    return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 4) & 1);
  }
}

}  // namespace park
