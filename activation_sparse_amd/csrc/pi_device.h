// pi_device.h - device helpers shared by the libpi kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pi {

constexpr int kWave = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// Elements carried by one 16-byte vector of a row, per storage type.
template <int DT> struct Fmt;
template <> struct Fmt<0> { static constexpr int E = 4; };   // fp32
template <> struct Fmt<1> { static constexpr int E = 8; };   // fp16
template <> struct Fmt<2> { static constexpr int E = 32; };  // int4, group 128

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float h2f(uint16_t bits) {
  _Float16 h = __builtin_bit_cast(_Float16, bits);
  return (float)h;
}

// Widen one 16-byte vector into E floats.  For int4 `scale` multiplies each
// signed nibble (even element in the low nibble).
template <int DT>
__device__ __forceinline__ void widen(const uint4 v, float scale, float* out) {
  if constexpr (DT == 0) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  } else if constexpr (DT == 1) {
    half8 h = __builtin_bit_cast(half8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (float)h[i];
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        int q = (int)((w[i] >> (4 * n)) & 0xF);
        q = (q ^ 8) - 8;  // sign-extend the nibble
        out[i * 8 + n] = (float)q * scale;
      }
    }
  }
}

// Row geometry: bytes per row and 16-byte vectors per row.
__host__ __device__ __forceinline__ int64_t row_bytes(int dt, int64_t cols) {
  return dt == 0 ? cols * 4 : dt == 1 ? cols * 2 : cols / 2;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float load_bias(const void* p, int dt, int64_t i) {
  if (!p) return 0.f;
  return dt == 0 ? reinterpret_cast<const float*>(p)[i] : h2f(reinterpret_cast<const uint16_t*>(p)[i]);
}

}  // namespace pi
