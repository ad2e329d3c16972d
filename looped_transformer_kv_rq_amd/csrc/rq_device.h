// Device helpers shared by the librq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 bf16 (one 16-byte load) -> 8 floats
__device__ __forceinline__ void bf16x8_to_f32(const uint4 u, float* f) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

// 32 consecutive bf16 (64 bytes, 16-byte aligned) -> 32 floats
__device__ __forceinline__ void load_bf16x32(const uint16_t* p, float (&f)[32]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) bf16x8_to_f32(q[i], f + 8 * i);
}

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// float -> fp16 bits, round to nearest even, saturated at +-65504
__device__ __forceinline__ uint16_t f32_to_f16_sat(float x) {
  x = fminf(fmaxf(x, -65504.0f), 65504.0f);
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Value of the lane whose index differs in bit log2(MASK), for MASK in {1, 2}
// (DPP quad_perm: stays inside a quad of lanes).
template <int MASK>
__device__ __forceinline__ float quad_xor(float v) {
  static_assert(MASK == 1 || MASK == 2, "quad_xor covers lane bits 0 and 1");
  constexpr int ctrl = MASK == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, true));
}

// Unnormalised in-register Walsh-Hadamard transform of 32 values (natural
// order): the butterflies on index bits 0..4.
__device__ __forceinline__ void fwht32(float (&y)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
    }
  }
}

// Butterfly on the index bit held by lane bit log2(MASK): the lane owning the
// lower half keeps a + b, the upper one a - b.
template <int MASK>
__device__ __forceinline__ void fwht_xlane(float (&y)[32], bool upper) {
  const float sgn = upper ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float p = quad_xor<MASK>(y[i]);
    y[i] = fmaf(sgn, y[i], p);
  }
}

// Full unnormalised transform of a head_dim vector spread as one 32-value
// group per lane over D/32 consecutive lanes (lane g holds coordinates
// [32g, 32g+32)).
template <int D>
__device__ __forceinline__ void fwht_groups(float (&y)[32], int g) {
  fwht32(y);
  if constexpr (D >= 64) fwht_xlane<1>(y, (g & 1) != 0);
  if constexpr (D >= 128) fwht_xlane<2>(y, (g & 2) != 0);
}

template <int D>
struct RsqrtD;
template <>
struct RsqrtD<64> { static constexpr float v = 0.125f; };
template <>
struct RsqrtD<128> { static constexpr float v = 0.08838834764831845f; };

}  // namespace rq
