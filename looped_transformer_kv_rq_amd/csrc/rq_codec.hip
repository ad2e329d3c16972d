// ResidualQuant encode and reconstruct kernels for gfx950.
//
// Encode (ResidualQuant, newx.sg page, Abstract): each earlier loop's K or V is
// stored as a residual against the final loop. The residual is rotated, given
// a least-squares scale per group and stored with 2 or 4 bits per coordinate.
//
// Work layout: a head_dim vector is handled by D/32 consecutive lanes, and
// lane g holds coordinates [32g, 32g+32). The Walsh-Hadamard butterflies on
// index bits 0..4 stay in registers, and the one or two butterflies on the
// higher bits go across lanes inside a quad (DPP). After the transform, each
// lane owns exactly one 32-coordinate scale group. The absmax, the code
// assignment, the least-squares fit and the packing then need no lane
// exchange. Loads are 16 bytes per instruction, and a quad covers one
// contiguous 256-byte vector. Stores are contiguous across a quad: 8 or 16
// bytes of codes per lane, and one fp16 scale per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

template <int BITS>
struct Grid {
  static constexpr int kHalf = 1 << (BITS - 1);      // code of level +1/2
  static constexpr int kTop = (1 << BITS) - 1;
  static constexpr float kOff = kHalf - 0.5f;         // level = code - kOff
  static constexpr int kPerWord = 32 / BITS;          // codes per uint32
};

// Quantize one rotated group (unnormalised transform values y' = sqrt(D) y)
// and store its packed codes and fp16 scale. Codes are invariant to the
// common sqrt(D) factor; the scale is divided by it at the end.
template <int BITS, int D>
__device__ __forceinline__ void quantize_group_store(const float (&y)[32], uint32_t* __restrict__ codes,
                                                     uint16_t* __restrict__ scales, int64_t v, int g) {
  using G = Grid<BITS>;
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(y[i]));

  uint32_t words[BITS];
#pragma unroll
  for (int k = 0; k < BITS; ++k) words[k] = 0u;
  float s = 0.0f;
  if (m > 0.0f) {
    const float inv = G::kOff / m;  // 1 / s0
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float c = fminf(fmaxf(floorf(y[i] * inv) + (float)G::kHalf, 0.0f), (float)G::kTop);
      const float q = c - G::kOff;
      num = fmaf(y[i], q, num);
      den = fmaf(q, q, den);
      words[i / G::kPerWord] |= (uint32_t)c << (BITS * (i % G::kPerWord));
    }
    s = num / den * RsqrtD<D>::v;
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) words[i / G::kPerWord] |= (uint32_t)G::kHalf << (BITS * (i % G::kPerWord));
  }
  uint32_t* dst = codes + v * (D * BITS / 32) + g * BITS;
  if constexpr (BITS == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
  } else {
    *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
  }
  scales[v * (D / 32) + g] = f32_to_f16_sat(s);
}

template <int D>
__global__ __launch_bounds__(256) void rq_encode_kernel(EncodeArgs a) {
  constexpr int kLanes = D / 32;      // lanes per vector
  constexpr int kVecPerBlock = 256 / kLanes;
  const int g = threadIdx.x % kLanes;
  const int64_t stride = (int64_t)gridDim.x * kVecPerBlock;
  for (int64_t v = (int64_t)blockIdx.x * kVecPerBlock + threadIdx.x / kLanes; v < a.n_vec; v += stride) {
    const int64_t base = v * D + g * 32;
    float ref[32];
    load_bf16x32(a.ref + base, ref);
    for (int l = 0; l < a.n_loops; ++l) {
      float y[32];
      load_bf16x32(a.x[l] + base, y);
#pragma unroll
      for (int i = 0; i < 32; ++i) y[i] -= ref[i];
      fwht_groups<D>(y, g);
      if (a.bits[l] == 2) {
        quantize_group_store<2, D>(y, a.codes[l], a.scales[l], v, g);
      } else {
        quantize_group_store<4, D>(y, a.codes[l], a.scales[l], v, g);
      }
    }
  }
}

template <int D, int BITS, bool BF16OUT>
__global__ __launch_bounds__(256) void rq_reconstruct_kernel(ReconstructArgs a) {
  constexpr int kLanes = D / 32;
  constexpr int kVecPerBlock = 256 / kLanes;
  const int g = threadIdx.x % kLanes;
  const int64_t stride = (int64_t)gridDim.x * kVecPerBlock;
  for (int64_t v = (int64_t)blockIdx.x * kVecPerBlock + threadIdx.x / kLanes; v < a.n_vec; v += stride) {
    const int64_t base = v * D + g * 32;
    float x[32];
    load_bf16x32(a.ref + base, x);
    if constexpr (BITS != 0) {
      using G = Grid<BITS>;
      const float s = f16_bits_to_f32(a.scales[v * (D / 32) + g]) * RsqrtD<D>::v;
      const uint32_t* src = a.codes + v * (D * BITS / 32) + g * BITS;
      uint32_t words[BITS];
      if constexpr (BITS == 2) {
        const uint2 w = *reinterpret_cast<const uint2*>(src);
        words[0] = w.x; words[1] = w.y;
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(src);
        words[0] = w.x; words[1] = w.y; words[2] = w.z; words[3] = w.w;
      }
      float z[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t c = (words[i / G::kPerWord] >> (BITS * (i % G::kPerWord))) & (uint32_t)G::kTop;
        z[i] = s * ((float)c - G::kOff);
      }
      fwht_groups<D>(z, g);
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] += z[i];
    } else {
      (void)g;
    }
    if constexpr (BF16OUT) {
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + base);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 u;
        u.x = f32_to_bf16_bits(x[8 * i + 0]) | (f32_to_bf16_bits(x[8 * i + 1]) << 16);
        u.y = f32_to_bf16_bits(x[8 * i + 2]) | (f32_to_bf16_bits(x[8 * i + 3]) << 16);
        u.z = f32_to_bf16_bits(x[8 * i + 4]) | (f32_to_bf16_bits(x[8 * i + 5]) << 16);
        u.w = f32_to_bf16_bits(x[8 * i + 6]) | (f32_to_bf16_bits(x[8 * i + 7]) << 16);
        dst[i] = u;
      }
    } else {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + base);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
    }
  }
}

static unsigned grid_for(int64_t n_vec, int vec_per_block) {
  int64_t blocks = (n_vec + vec_per_block - 1) / vec_per_block;
  const int64_t cap = 1 << 20;  // grid-stride beyond this
  if (blocks > cap) blocks = cap;
  return (unsigned)(blocks < 1 ? 1 : blocks);
}

hipError_t launch_encode(const EncodeArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 128) {
    hipLaunchKernelGGL(rq_encode_kernel<128>, dim3(grid_for(a.n_vec, 64)), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(rq_encode_kernel<64>, dim3(grid_for(a.n_vec, 128)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D>
static void launch_reconstruct_d(const ReconstructArgs& a, int bits, int out_bf16, hipStream_t stream) {
  const dim3 grid(grid_for(a.n_vec, 256 / (D / 32))), block(256);
#define RQ_RECON(B, O) hipLaunchKernelGGL((rq_reconstruct_kernel<D, B, O>), grid, block, 0, stream, a)
  if (bits == 0) {
    if (out_bf16) RQ_RECON(0, true); else RQ_RECON(0, false);
  } else if (bits == 2) {
    if (out_bf16) RQ_RECON(2, true); else RQ_RECON(2, false);
  } else {
    if (out_bf16) RQ_RECON(4, true); else RQ_RECON(4, false);
  }
#undef RQ_RECON
}

hipError_t launch_reconstruct(const ReconstructArgs& a, int head_dim, int bits, int out_bf16, hipStream_t stream) {
  if (head_dim == 128) launch_reconstruct_d<128>(a, bits, out_bf16, stream);
  else launch_reconstruct_d<64>(a, bits, out_bf16, stream);
  return hipGetLastError();
}

}  // namespace rq
