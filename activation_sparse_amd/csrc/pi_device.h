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

// Buffer resources: a wave-uniform base, a byte range, and loads at 32-bit
// offsets from it.  A load whose 16 (or 2) bytes lie past the range returns
// zeros and issues no memory request, so lanes past a row's end need neither
// a clamped address nor a branch.  Word 3 is the gfx9-family default
// (untyped, no swizzle).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t bload2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
// A pointer every lane of the wave holds, moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
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

// DPP move within a 16-lane row (CTRL: row_ror:n = 0x120 + n).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each 16-lane row, returned in every lane of the row (rotations by
// 8, 4, 2, 1; each lane's association order is fixed).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0x128>(v);
  v += dpp_mov<0x124>(v);
  v += dpp_mov<0x122>(v);
  v += dpp_mov<0x121>(v);
  return v;
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes of a wave, wave-uniform, in a fixed order: the four
// row sums (lanes 0, 16, 32, 48) added pairwise.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

__device__ __forceinline__ float load_bias(const void* p, int dt, int64_t i) {
  if (!p) return 0.f;
  return dt == 0 ? reinterpret_cast<const float*>(p)[i] : h2f(reinterpret_cast<const uint16_t*>(p)[i]);
}

// Bias access for a bias dtype fixed at compile time (BDT: 0 fp32, 1 fp16)
// through a buffer resource over its n entries: an absent bias (NULL) is an
// empty range, which reads zeros.  Buffer loads keep the vmcnt order exact, so
// a bias issued before a row's weights is usable without waiting for them.
template <int BDT>
struct Bias {
  rsrc_t r;
  __device__ __forceinline__ Bias(const void* q, uint32_t n)
      : r(make_rsrc(uniform_ptr(q), q ? n * (BDT == 0 ? 4u : 2u) : 0u)) {}
  __device__ __forceinline__ float operator()(int64_t i) const {
    if constexpr (BDT == 0) return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)(i * 4), 0, 0));
    else return h2f(bload2(r, (uint32_t)i * 2u));
  }
};

}  // namespace pi
