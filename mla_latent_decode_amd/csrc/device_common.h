// Device helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkmla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define QK_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))
#define QK_GLB(T, p) ((__attribute__((address_space(1))) T*)(p))

// Storage element <-> float.  bf16 is kept as raw 16-bit words in memory.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
// Round to nearest, ties to even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// cos and sin of the RoPE angle p * base^(-2i/d).  The angle is formed and
// reduced modulo 2*pi in double, so positions up to 2^18 keep full float
// accuracy; the reduced angle goes through float sincos.
__device__ __forceinline__ void rope_cos_sin(int pos, int i, int d, float base, float* c,
                                             float* s) {
  const double two_pi = 6.283185307179586476925286766559;
  double ang = (double)pos * pow((double)base, -2.0 * (double)i / (double)d);
  ang -= two_pi * floor(ang / two_pi);
  sincosf((float)ang, s, c);
}

// cos and sin of pos * freq, freq one of the host's RoPE frequencies
// (RopeFreq): the angle is formed and reduced modulo 2*pi in double (exact to
// about 2^-35 rad for positions below 2^18), then float sincos.
__device__ __forceinline__ void rope_cos_sin_freq(int pos, double freq, float* c, float* s) {
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  const double ang = (double)pos * freq;
  const double red = fma(-floor(ang * inv_two_pi), two_pi, ang);
  sincosf((float)red, s, c);
}

// Sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace qkmla
