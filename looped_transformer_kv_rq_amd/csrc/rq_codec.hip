// ResidualQuant encode and reconstruct kernels for gfx950.
//
// Encode (ResidualQuant, newx.sg page, Abstract): each earlier loop's K or V is
// stored as a residual against the final loop. The residual is rotated, given
// a least-squares scale per group and stored with 2 or 4 bits per coordinate
// (3 or 8 for a per-(layer, loop) table; AI Summary: layer-wise precision).
//
// Code words of one vector (W = D b / 32 of them):
//  * b in {2, 4, 8}: word w holds coordinates [(32/b) w, (32/b)(w+1)), the
//    coordinate j of the word at bits [b j, b j + b);
//  * b = 3: two bit planes, so no code crosses a word. Words [0, D/16) hold
//    the low two bits of every code in the INT2 layout, words [D/16, 3D/32)
//    bit 2 of every code (coordinate j of word w at bit j).
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
  static constexpr int kPerWord = 32 / BITS;          // codes per uint32 (b = 2, 4, 8)
};

// Code of coordinate i (0..31) of a group from its BITS packed words (for
// b = 3: the two INT2-plane words, then the bit-2 word).
template <int BITS>
__device__ __forceinline__ uint32_t group_code(const uint32_t (&words)[BITS], int i) {
  if constexpr (BITS == 3) {
    return ((words[i / 16] >> (2 * (i % 16))) & 3u) | (((words[2] >> i) & 1u) << 2);
  } else {
    using G = Grid<BITS>;
    return (words[i / G::kPerWord] >> (BITS * (i % G::kPerWord))) & (uint32_t)G::kTop;
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// x_lo * c_lo + x_hi * c_hi + acc over one pair of bf16 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t c, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), __builtin_bit_cast(bf16x2_t, c), acc,
                                         false);
}
constexpr uint32_t kPairSum = 0x3F803F80u;   // bf16 (+1, +1)
constexpr uint32_t kPairDiff = 0xBF803F80u;  // bf16 (+1, -1), low half first

// Quantize one rotated group (unnormalised transform values y' = sqrt(D) y)
// and return its packed code words and the scale. Codes are invariant to the
// common sqrt(D) factor; the scale is divided by it at the end.
//  * c = floor(y / s0) + 2^(b-1) with 1 / s0 = (2^(b-1) - 1/2) / max|y|. For
//    finite inputs |y / s0| <= 2^(b-1) - 1/2, so c already lies in
//    [0, 2^b - 1] and needs no clamp. An all-zero group takes 1 / s0 = 0,
//    which gives every code 2^(b-1) and num = 0, so s = 0.
//  * Packing sums c * 2^(b i) in fp32 over 16-bit halves of a word (exact:
//    every partial sum is an integer below 2^16). INT3 packs its two planes
//    with integer shifts.
//  * INT2: q^2 is 1/4 for the inner codes 1, 2 and 9/4 for 0, 3, so
//    <q, q> = 72 - 2 * (number of inner codes), counted on the packed words.
//  * refits > 0 alternates the two least-squares half-steps that many more
//    times: codes at the current scale (same floor rule, now clamped to the
//    grid, since |y| / s may exceed the top level), then the LS scale again.
template <int BITS, int D, bool REFIT>
__device__ __forceinline__ float quantize_group(const float* y, int refits, uint32_t (&words)[BITS]) {
  using G = Grid<BITS>;
  constexpr int kPerHalf = BITS == 3 ? 1 : G::kPerWord / 2;  // codes per 16-bit half word
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(y[i]));
  float inv = m > 0.0f ? G::kOff / m : 0.0f;  // 1 / step of the assignment
  float sfit = 0.0f;
  const int passes = REFIT ? refits + 1 : 1;
  for (int pass = 0; pass < passes; ++pass) {
    float num = 0.0f, den = 0.0f;
    float half[2 * BITS];
#pragma unroll
    for (int k = 0; k < 2 * BITS; ++k) half[k] = 0.0f;
    uint32_t plane[3] = {0u, 0u, 0u};  // INT3: low-bit words, bit-2 word
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      // (no clamp is needed at the absmax step; the refit steps clamp)
      float c = floorf(fmaf(y[i], inv, (float)G::kHalf));
      if constexpr (REFIT) c = __builtin_amdgcn_fmed3f(c, 0.0f, (float)G::kTop);
      const float q = c - G::kOff;
      num = fmaf(y[i], q, num);
      if constexpr (BITS != 2) den = fmaf(q, q, den);
      if constexpr (BITS == 3) {
        const uint32_t ci = (uint32_t)c;
        plane[i / 16] |= (ci & 3u) << (2 * (i % 16));
        plane[2] |= (ci >> 2) << i;
      } else {
        half[i / kPerHalf] = fmaf(c, (float)(1u << (BITS * (i % kPerHalf))), half[i / kPerHalf]);
      }
    }
    if constexpr (BITS == 3) {
#pragma unroll
      for (int k = 0; k < 3; ++k) words[k] = plane[k];
    } else {
#pragma unroll
      for (int k = 0; k < BITS; ++k)
        words[k] = (uint32_t)half[2 * k] | ((uint32_t)half[2 * k + 1] << 16);
    }
    if constexpr (BITS == 2) {
      int inner = 0;
#pragma unroll
      for (int k = 0; k < 2; ++k) inner += __builtin_popcount((words[k] ^ (words[k] >> 1)) & 0x55555555u);
      den = (float)(72 - 2 * inner);
    }
    sfit = num / den;                       // 0 for an all-zero group
    inv = sfit > 0.0f ? 1.0f / sfit : 0.0f;  // step of the next assignment
  }
  return sfit * RsqrtD<D>::v;
}

// Encode kernel: PER coordinates of a vector per lane (PER / 32 scale
// groups), D / PER consecutive lanes per vector.
//  * The first butterfly (index bit 0) is folded into the bf16 unpacking:
//    for the pair (x0, x1) with reference (r0, r1), one dot2 instruction
//    gives (x0 - r0) + (x1 - r1) = x0 + x1 - (r0 + r1), and another the
//    difference; the reference pair sums are formed once for all loops.
//  * Butterflies on the remaining in-lane index bits stay in registers; those
//    on the lane bits go across lanes inside a quad (DPP).
//  * WIDE instantiations also take INT3 and INT8 loops; the INT2/INT4-only
//    ones carry no code for them.
// SETS: tensors of the launch (1, or 2 for K and V together); blockIdx.y
// picks the tensor.
template <int D, int PER, bool REFIT, bool APPEND, bool WIDE, int SETS>
__global__ __launch_bounds__(256) void rq_encode_kernel(EncodeLaunch launch) {
  const EncodeArgs& a = launch.set[SETS == 1 ? 0 : blockIdx.y];
  constexpr int kLanes = D / PER;  // lanes per vector
  constexpr int kVecPerBlock = 256 / kLanes;
  constexpr int NGL = PER / 32;    // scale groups per lane
  const int sub = threadIdx.x % kLanes;
  const int64_t stride = (int64_t)gridDim.x * kVecPerBlock;
  for (int64_t v = (int64_t)blockIdx.x * kVecPerBlock + threadIdx.x / kLanes; v < a.n_vec; v += stride) {
    const int64_t base = v * D + sub * PER;
    // Output vector. Appending: source vector (row, t) of a [rows][t_new] batch
    // goes to cache position pos[b] + t of row = b * Hkv + h; a position past the
    // cache's capacity (or a negative one) writes nothing. In a paged cache the
    // position lives in block block_table[b][p / P] at offset p % P; a position
    // whose table entry is not a valid block writes nothing either.
    int64_t vo = v;
    if constexpr (APPEND) {
      const int64_t row = v / a.t_new;
      const int64_t bq = row / a.n_kv_heads;
      const int64_t p = (int64_t)a.pos[bq] + v % a.t_new;
      if (p < 0 || p >= a.s_cap) continue;  // uniform across the vector's lanes
      if (a.block_table != nullptr) {
        const int blk = a.block_table[bq * a.max_blocks + (p >> a.log2_block)];
        if (blk < 0 || blk >= a.n_blocks) continue;
        vo = (((int64_t)blk * a.n_kv_heads + row % a.n_kv_heads) << a.log2_block) +
             (p & ((1 << a.log2_block) - 1));
      } else {
        vo = row * a.s_cap + p;
      }
    }
    // negated reference pair sums and differences (zero without a reference)
    float nrs[PER / 2], nrd[PER / 2];
#pragma unroll
    for (int j = 0; j < PER / 2; ++j) nrs[j] = nrd[j] = 0.0f;
    if (a.ref != nullptr) {
      const uint4* rp = reinterpret_cast<const uint4*>(a.ref + base);
      uint4* rcopy = APPEND ? reinterpret_cast<uint4*>(a.ref_out + vo * D + sub * PER) : nullptr;
#pragma unroll
      for (int i = 0; i < PER / 8; ++i) {
        const uint4 u = rp[i];
        if (rcopy != nullptr) rcopy[i] = u;  // the final-loop state joins the reference cache
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float r0 = bf16_lo(w[j]), r1 = bf16_hi(w[j]);
          nrs[4 * i + j] = -(r0 + r1);
          nrd[4 * i + j] = r1 - r0;
        }
      }
    }
    for (int l = 0; l < a.n_loops; ++l) {
      float y[PER];
      const uint4* xp = reinterpret_cast<const uint4*>(a.x[l] + base);
#pragma unroll
      for (int i = 0; i < PER / 8; ++i) {
        const uint4 u = xp[i];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[8 * i + 2 * j] = dot2_bf16(w[j], kPairSum, nrs[4 * i + j]);
          y[8 * i + 2 * j + 1] = dot2_bf16(w[j], kPairDiff, nrd[4 * i + j]);
        }
      }
#pragma unroll
      for (int h = 2; h < PER; h <<= 1) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          if ((i & h) == 0) {
            const float p = y[i], q = y[i + h];
            y[i] = p + q;
            y[i + h] = p - q;
          }
        }
      }
      if constexpr (kLanes >= 2) {
        const float sgn = (sub & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < PER; ++i) y[i] = fmaf(sgn, y[i], quad_xor<1>(y[i]));
      }
      if constexpr (kLanes >= 4) {
        const float sgn = (sub & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < PER; ++i) y[i] = fmaf(sgn, y[i], quad_xor<2>(y[i]));
      }
      const int bits = a.bits[l];
      uint16_t sc[NGL];
      // INT2/INT4 codes and their scales go out as non-temporal stores: a
      // wave's store covers whole lines, nothing in the call reads them back,
      // and on MI355X the hint took about 6% off back-to-back encodes (the
      // previous launch's written lines no longer drain during the next one).
      if (bits == 2) {
        uint32_t wd[2 * NGL];
#pragma unroll
        for (int gi = 0; gi < NGL; ++gi) {
          uint32_t w2[2];
          sc[gi] = f32_to_f16_sat(quantize_group<2, D, REFIT>(y + 32 * gi, a.refits, w2));
          wd[2 * gi] = w2[0];
          wd[2 * gi + 1] = w2[1];
        }
        uint32_t* dst = a.codes[l] + vo * (D / 16) + sub * 2 * NGL;
        if constexpr (NGL == 2) __builtin_nontemporal_store(u32x4_t{wd[0], wd[1], wd[2], wd[3]}, reinterpret_cast<u32x4_t*>(dst));
        else __builtin_nontemporal_store(u32x2_t{wd[0], wd[1]}, reinterpret_cast<u32x2_t*>(dst));
      } else if (WIDE && bits == 3) {
        // low-bit plane at word 2g of the vector, bit-2 plane at word D/16 + g
        uint32_t* vec = a.codes[l] + vo * (3 * D / 32);
#pragma unroll
        for (int gi = 0; gi < NGL; ++gi) {
          uint32_t w3[3];
          sc[gi] = f32_to_f16_sat(quantize_group<3, D, REFIT>(y + 32 * gi, a.refits, w3));
          const int grp = sub * NGL + gi;
          *reinterpret_cast<uint2*>(vec + 2 * grp) = make_uint2(w3[0], w3[1]);
          vec[D / 16 + grp] = w3[2];
        }
      } else if (WIDE && bits == 8) {
        uint4* dst = reinterpret_cast<uint4*>(a.codes[l] + vo * (D / 4) + sub * 8 * NGL);
#pragma unroll
        for (int gi = 0; gi < NGL; ++gi) {
          uint32_t w8[8];
          sc[gi] = f32_to_f16_sat(quantize_group<8, D, REFIT>(y + 32 * gi, a.refits, w8));
          dst[2 * gi] = make_uint4(w8[0], w8[1], w8[2], w8[3]);
          dst[2 * gi + 1] = make_uint4(w8[4], w8[5], w8[6], w8[7]);
        }
      } else {
        uint32_t wd[4 * NGL];
#pragma unroll
        for (int gi = 0; gi < NGL; ++gi) {
          uint32_t w4[4];
          sc[gi] = f32_to_f16_sat(quantize_group<4, D, REFIT>(y + 32 * gi, a.refits, w4));
#pragma unroll
          for (int k = 0; k < 4; ++k) wd[4 * gi + k] = w4[k];
        }
        uint4* dst = reinterpret_cast<uint4*>(a.codes[l] + vo * (D / 8) + sub * 4 * NGL);
#pragma unroll
        for (int gi = 0; gi < NGL; ++gi) dst[gi] = make_uint4(wd[4 * gi], wd[4 * gi + 1], wd[4 * gi + 2], wd[4 * gi + 3]);
      }
      uint16_t* sdst = a.scales[l] + vo * (D / 32) + sub * NGL;
      if constexpr (NGL == 2) __builtin_nontemporal_store((uint32_t)sc[0] | ((uint32_t)sc[1] << 16), reinterpret_cast<uint32_t*>(sdst));
      else __builtin_nontemporal_store(sc[0], sdst);
    }
  }
}

// Reconstruct kernel: one scale group per lane, as in the encoder. A wave's
// 64 groups are 64 / (D / 32) whole vectors, contiguous in the output, so the
// wave stages its results in LDS (padded per lane against bank conflicts) and
// writes them back as contiguous 1 KB stores. Measured on MI355X, stores of
// each lane's own 128-byte run, spread over the wave's 8 KB, took 106 us
// against 68 us for one INT2 loop of l4_b16_s4k to fp32.
template <int D, int BITS, bool BF16OUT>
__global__ __launch_bounds__(256) void rq_reconstruct_kernel(ReconstructArgs a) {
  constexpr int kLanes = D / 32;
  constexpr int kVecPerBlock = 256 / kLanes;
  constexpr int kVecPerWave = 64 / kLanes;
  constexpr int kPad = BF16OUT ? 20 : 36;  // staged words per lane (32 values + padding)
  __shared__ __align__(16) uint32_t stage[4][64 * kPad];
  const int g = threadIdx.x % kLanes;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * kVecPerBlock;
  for (int64_t v0 = (int64_t)blockIdx.x * kVecPerBlock + wave * kVecPerWave; v0 < a.n_vec; v0 += stride) {
    // lanes past the last vector recompute it (the cross-lane butterflies need
    // every lane) and store nothing
    const int64_t v = min(v0 + lane / kLanes, a.n_vec - 1);
    const int64_t base = v * D + g * 32;
    float x[32];
    if (a.ref != nullptr) {
      load_bf16x32(a.ref + base, x);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = 0.0f;
    }
    if constexpr (BITS != 0) {
      using G = Grid<BITS>;
      const float s = f16_bits_to_f32(a.scales[v * (D / 32) + g]) * RsqrtD<D>::v;
      const uint32_t* vec = a.codes + v * (D * BITS / 32);
      uint32_t words[BITS];
      if constexpr (BITS == 2) {
        const uint2 w = *reinterpret_cast<const uint2*>(vec + 2 * g);
        words[0] = w.x; words[1] = w.y;
      } else if constexpr (BITS == 3) {
        const uint2 w = *reinterpret_cast<const uint2*>(vec + 2 * g);
        words[0] = w.x; words[1] = w.y; words[2] = vec[D / 16 + g];
      } else {
#pragma unroll
        for (int k = 0; k < BITS / 4; ++k) {
          const uint4 w = *reinterpret_cast<const uint4*>(vec + BITS * g + 4 * k);
          words[4 * k] = w.x; words[4 * k + 1] = w.y; words[4 * k + 2] = w.z; words[4 * k + 3] = w.w;
        }
      }
      float z[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) z[i] = s * ((float)group_code<BITS>(words, i) - G::kOff);
      fwht_groups<D>(z, g);
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] += z[i];
    } else {
      (void)g;
    }
    uint32_t* st = &stage[wave][lane * kPad];
    if constexpr (BF16OUT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 u;
        u.x = f32_to_bf16_bits(x[8 * i + 0]) | (f32_to_bf16_bits(x[8 * i + 1]) << 16);
        u.y = f32_to_bf16_bits(x[8 * i + 2]) | (f32_to_bf16_bits(x[8 * i + 3]) << 16);
        u.z = f32_to_bf16_bits(x[8 * i + 4]) | (f32_to_bf16_bits(x[8 * i + 5]) << 16);
        u.w = f32_to_bf16_bits(x[8 * i + 6]) | (f32_to_bf16_bits(x[8 * i + 7]) << 16);
        *reinterpret_cast<uint4*>(st + 4 * i) = u;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint4*>(st + 4 * i) = make_uint4(__float_as_uint(x[4 * i]), __float_as_uint(x[4 * i + 1]),
                                                           __float_as_uint(x[4 * i + 2]), __float_as_uint(x[4 * i + 3]));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the wave's vectors are contiguous in the output: 64 lanes x 32 values
    constexpr int kWords = BF16OUT ? 16 : 32;  // 32-bit words per lane chunk
    const int64_t n_words = min((int64_t)64 * kWords, (a.n_vec - v0) * D * kWords / 32);
    uint32_t* out = static_cast<uint32_t*>(a.out) + v0 * D * kWords / 32;
#pragma unroll
    for (int i = 0; i < kWords / 4; ++i) {
      const int e = 4 * lane + 256 * i;
      const uint4 u = *reinterpret_cast<const uint4*>(&stage[wave][(e / kWords) * kPad + e % kWords]);
      if (e < n_words) *reinterpret_cast<uint4*>(out + e) = u;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

static unsigned grid_for(int64_t n_vec, int vec_per_block) {
  int64_t blocks = (n_vec + vec_per_block - 1) / vec_per_block;
  const int64_t cap = 1 << 20;  // grid-stride beyond this
  if (blocks > cap) blocks = cap;
  return (unsigned)(blocks < 1 ? 1 : blocks);
}

// 32 coordinates (one scale group) per lane: measured on MI355X, 64 per lane
// saves the second cross-lane butterfly but halves the occupancy (about 200
// registers) and runs slower.
constexpr int kEncodePer = 32;

template <int D, bool WIDE, int SETS>
static void launch_encode_dw(const EncodeLaunch& l, hipStream_t stream) {
  constexpr int per = kEncodePer;
  const EncodeArgs& a = l.set[0];
  const dim3 grid(grid_for(a.n_vec, 256 / (D / per)), SETS);
  if (a.pos != nullptr)
    hipLaunchKernelGGL((rq_encode_kernel<D, per, false, true, WIDE, SETS>), grid, dim3(256), 0, stream, l);
  else if (a.refits > 0)
    hipLaunchKernelGGL((rq_encode_kernel<D, per, true, false, WIDE, SETS>), grid, dim3(256), 0, stream, l);
  else
    hipLaunchKernelGGL((rq_encode_kernel<D, per, false, false, WIDE, SETS>), grid, dim3(256), 0, stream, l);
}

template <int D>
static void launch_encode_d(const EncodeLaunch& l, int n_sets, hipStream_t stream) {
  bool wide = false;
  for (int s = 0; s < n_sets; ++s)
    for (int i = 0; i < l.set[s].n_loops; ++i) wide = wide || l.set[s].bits[i] == 3 || l.set[s].bits[i] == 8;
  if (n_sets == 2) {
    if (wide) launch_encode_dw<D, true, 2>(l, stream);
    else launch_encode_dw<D, false, 2>(l, stream);
  } else {
    if (wide) launch_encode_dw<D, true, 1>(l, stream);
    else launch_encode_dw<D, false, 1>(l, stream);
  }
}

hipError_t launch_encode(const EncodeArgs* sets, int n_sets, int head_dim, hipStream_t stream) {
  if (n_sets < 1 || n_sets > kMaxEncodeSets) return hipErrorInvalidValue;
  for (int s = 1; s < n_sets; ++s) {  // one grid: the sets share the shape and the kind of launch
    if (sets[s].n_vec != sets[0].n_vec || (sets[s].pos == nullptr) != (sets[0].pos == nullptr) ||
        sets[s].refits != sets[0].refits)
      return hipErrorInvalidValue;
  }
  EncodeLaunch l{};
  for (int s = 0; s < n_sets; ++s) l.set[s] = sets[s];
  if (head_dim == 128) launch_encode_d<128>(l, n_sets, stream);
  else launch_encode_d<64>(l, n_sets, stream);
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
  } else if (bits == 3) {
    if (out_bf16) RQ_RECON(3, true); else RQ_RECON(3, false);
  } else if (bits == 4) {
    if (out_bf16) RQ_RECON(4, true); else RQ_RECON(4, false);
  } else {
    if (out_bf16) RQ_RECON(8, true); else RQ_RECON(8, false);
  }
#undef RQ_RECON
}

hipError_t launch_reconstruct(const ReconstructArgs& a, int head_dim, int bits, int out_bf16, hipStream_t stream) {
  if (head_dim == 128) launch_reconstruct_d<128>(a, bits, out_bf16, stream);
  else launch_reconstruct_d<64>(a, bits, out_bf16, stream);
  return hipGetLastError();
}

}  // namespace rq
