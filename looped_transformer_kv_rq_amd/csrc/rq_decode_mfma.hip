// Split-S decode attention over the ResidualQuant cache on gfx950 matrix cores.
//
// ResidualQuant (newx.sg page, Abstract): an earlier loop's K/V is the bf16
// final-loop reference plus a rotated INT2/INT4 residual with a least-squares
// fp16 scale per 32 coordinates (INT3/INT8 too for a per-(layer, loop) table,
// AI Summary). One call attends every loop's queries over
// the cache and streams the reference once for all of them. The rotation H
// (normalised Walsh-Hadamard) is symmetric, so
//   score  = q . k_ref + (H q) . (s * lev)
//   output = sum_t p_t v_ref,t + H sum_t p_t (s * lev)_t.
// The query is rotated once per block by the partial kernel itself (or, for the
// launches that cannot, once per call by rq_query_prep). The partial kernel
// keeps the residual terms in the rotated domain, and the combine kernel
// applies H to the merged residual accumulator of each query row once.
//
// Partial kernel: one block is four independent waves over one split of one
// (batch, kv head) row. A wave takes 32-token tiles (tiles w, w+4, ...). Every
// query row of the kv head (loops x G query heads, at most 32 = two 16-row
// blocks) is one MFMA column. A launch with more than 16 rows whose loops fit
// 16 each runs as two argument sets of one 16-row block, paired: a block is
// then two waves, one per set, that walk the same tiles and share each tile's
// reference K and V through LDS. All products run on v_mfma_f32_16x16x32:
//  * reference scores S^T = K_ref Q^T (bf16; exact products, fp32 sums). The
//    K tile is loaded straight into the A operand;
//  * residual scores per loop and scale group (fp16), two products: one with
//    the hi and one with the lo half of the rotated query (hi + lo carries it
//    to about 2^-22). A code becomes the fp16 value 1 + c / 2^b when it is
//    masked into the mantissa of 1.0. The per-row constant of that offset is
//    taken out afterwards: q . (c - o) = 2^b (q . val) - (2^b + o) sum(q);
//  * reference PV, O_ref^T += V^T P^T (bf16). P is split into bf16 hi + lo
//    halves (error ~2^-16), and V^T is read from the LDS tile;
//  * residual PV, O_res^T += lev^T (P s)^T (fp16; each weight P s is the
//    fp32 P times the fp16 scale, rounded once to nearest). In 16-row blocks
//    INT2 and INT4 levels enter as the mantissa value 1 + c / 2^b, and one
//    more product with an operand of ones gives each group's sum of P s for
//    the offset, taken out once per row after the token loop. INT3 levels
//    (and every width in 32-row blocks) decode exactly through a v_perm byte
//    table; INT8 levels are formed as 2 lev = (1024 + 2c) - 1279 in fp16
//    against P s / 2. Rows of other loops carry P s = 0, so every loop shares
//    one accumulator.
// The MFMA output layout (lane l holds rows 4 (l / 16) + i of column l % 16)
// gives each lane one query row and four tokens per 16-token block. The
// softmax statistics of a row therefore stay within the row's four lanes,
// and the P fragment is already the B operand of the PV products.
//
// Each tile's loads go out together at its start. The K reference goes to
// registers. The V tile and every residual loop's codes and scales go to LDS
// by DMA (global_load_lds). A tile therefore costs one memory round trip
// however many loops it carries.
//
// PAGED instantiations read a block-paged cache: each tensor is
// [n_blocks][Hkv][P][row] and position t of sequence b lives in block
// block_table[b][t / P] at offset t % P. P is a power of two and a multiple of
// 64, so a 32-token tile lies in one block and one table entry places it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ f32x4_t mma_bf16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma_f16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}
__device__ __forceinline__ uint32_t vperm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}
// fp16 pair {p0 * s0, p1 * s1} from fp32 weights p and fp16 scales taken from
// half `hi` of the words w0 and w1, each product rounded once to nearest even
// (v_fma_mixlo_f16 / v_fma_mixhi_f16 with a zero addend). Unbiased: the
// residual PV's weights then carry no systematic error.
__device__ __forceinline__ uint32_t mix_pair(float p0, uint32_t w0, float p1, uint32_t w1, bool hi) {
  uint32_t r;
  if (hi) {
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p0), "v"(w0));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(r) : "v"(p1), "v"(w1));
  } else {
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p0), "v"(w0));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(r) : "v"(p1), "v"(w1));
  }
  return r;
}
// Maximum of v over lanes l, l^16, l^32 and l^48 (a row's four lane groups),
// by the gfx950 row-swap permutes: with both operands v, permlane16_swap gives
// each lane the values of its even and its odd 16-lane row, permlane32_swap
// those of its lower and upper 32-lane half. No LDS round trip on the softmax's
// path, as a bpermute shuffle would take.
__device__ __forceinline__ float max_xor16_32(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const uint32_t w = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// 2^x by v_exp_f32 alone (no denormal-range fix-up): softmax weights below
// 2^-126 of the running maximum count as zero. 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }

// LDS DMA (gfx950 global_load_lds): every active lane fetches `bytes` from its
// own global address; lane l's data lands at dst + l * bytes (dst uniform).
// The 16-byte forms carry the non-temporal hint (cache policy bit nt): each of
// their instructions reads whole 128-byte lines of data that is read once per
// call, and on MI355X the hint took about 4% off the l4_b16_s4k decode. The
// 4-byte forms keep the default policy, because the transposed V-code loads
// read a line in pieces over several instructions and a streamed line would
// be fetched again for each piece.
constexpr int kStreamPolicy = 2;  // nt
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, kStreamPolicy);
}
__device__ __forceinline__ void dma16_keep(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 4, 0, 0);
}
// Buffer-resource forms for tiles that lie inside the sequence: the resource
// (base = start of the (batch, kv head) row, set up in scalar registers) and
// the tile offset are wave-uniform, the per-lane offset is a constant, so
// issuing a tile costs no vector instructions.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, voff, soff, 0, kStreamPolicy);
}
__device__ __forceinline__ void bdma16_keep(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void bdma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// s_waitcnt vmcnt(0) / lgkmcnt(0) (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4], lgkmcnt [11:8])
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr uint32_t kLutInt2 = 0x3E38B8BEu;    // fp16 high bytes of -1.5, -0.5, 0.5, 1.5
constexpr uint32_t kLutInt4Hi = 0x4640C0C6u;  // fp16 high bytes of -6, -2, 2, 6 (4 * INT2 level)
constexpr uint32_t kLutInt3Lo = 0xB8BEC1C3u;  // fp16 high bytes of -3.5, -2.5, -1.5, -0.5
constexpr uint32_t kLutInt3Hi = 0x43413E38u;  // fp16 high bytes of 0.5, 1.5, 2.5, 3.5
constexpr int kTile = 32;
constexpr int kTile16 = 16;  // tokens per MFMA row block

// Residual accumulator blocks per 16-row block: 2 D/32 output blocks, and at
// NB = 1 one more per scale group for the weight sums of the INT2 / INT4
// decode (residual_pv). At NB = 2 those would push the kernel into spills, so
// it decodes every width through the byte table.
template <int D, int NB>
constexpr int kResBlocks = 2 * (D / 32) + (NB == 1 ? D / 32 : 0);

template <int D>
struct MfmaGeom {
  static constexpr int NG = D / 32;    // scale groups = k-steps of the score products
  static constexpr int NH = D / 64;    // 64-coordinate halves of the reference PV
  // V tile: one DMA instruction writes 1 KB (VT_TOK tokens); a 128-byte pad
  // after each keeps the transposed reads of neighbouring lane groups apart.
  static constexpr int VT_TOK = 1024 / (2 * D);
  static constexpr int VT_INSTR = kTile / VT_TOK;
  static constexpr int VT_STRIDE = 1024 + 128;
  static constexpr int VT_BYTES = VT_INSTR * VT_STRIDE;
  static __device__ __forceinline__ int vt_offset(int tok) {
    return (tok / VT_TOK) * VT_STRIDE + (tok % VT_TOK) * 2 * D;
  }
  // rotated query record: fp16 hi parts in operand order, then the fp16 lo
  // parts, then the per-group offsets
  static constexpr int PREP_BYTES = (4 * D + 4 * NG + 15) / 16 * 16;
};

// LDS bytes of one residual loop's tile data: K code words [token][W],
// K scales [token][NG], V code words transposed [word][token], V scales
__host__ __device__ constexpr int loop_lds_bytes(int d, int bits) {
  return bits == 0 ? 0 : 256 * (d * bits / 32) + 128 * (d / 32);
}

// K code words sit in LDS as [token][W] in 16-byte chunks. With SWZ the chunks
// of token t are rotated by ((t * W/4) >> 4) & min(W/4 - 1, 3) as the DMA lands
// them: the 16 tokens of one MFMA row block, each read at one chunk index,
// then fall on different LDS banks (on two at most for INT8 at head_dim 128).
// Unrotated, INT4 tokens m, m+4, m+8 and m+12 (and INT2 tokens m and m+8)
// share banks: 257 conflict cycles per tile and wave at mixed_s32k, against
// 1 rotated, and the decode 3% faster; INT8 tokens two apart share them
// (eight ways). The kernels with INT3 / INT8 loops, at their register limit,
// rotate only the INT8 loops (the 32-row ones not at all): the per-lane
// offsets of every width spill them.
template <int D, int BITS, bool SWZ>
constexpr int kKcSwz = SWZ && BITS != 3 ? (D * BITS / 128 - 1 < 3 ? D * BITS / 128 - 1 : 3) : 0;

// LDS offset of residual slot li's tile data inside a wave's buffer: the V
// tile, then the slots in the launcher's order INT8, INT4, INT3, INT2 (after
// the other set's slots in a paired launch, lds_res_base).
template <int D, bool WIDE>
__device__ __forceinline__ int slot_lds_offset(const DecodeArgs& a, int li) {
  constexpr int L4 = loop_lds_bytes(D, 4), L2 = loop_lds_bytes(D, 2);
  if constexpr (!WIDE) {
    return MfmaGeom<D>::VT_BYTES + a.lds_res_base + (li < a.n4 ? li * L4 : a.n4 * L4 + (li - a.n4) * L2);
  } else {
    constexpr int L8 = loop_lds_bytes(D, 8), L3 = loop_lds_bytes(D, 3);
    int off = MfmaGeom<D>::VT_BYTES + a.lds_res_base;
    int k = min(li, a.n8);
    off += k * L8;
    li -= k;
    k = min(li, a.n4);
    off += k * L4;
    li -= k;
    k = min(li, a.n3);
    off += k * L3;
    li -= k;
    return off + li * L2;
  }
}

// ---------------------------------------------------------------------------
// query prep: rotated query in residual-score B-operand order + offsets
// ---------------------------------------------------------------------------

// Coordinate that lane group g, k-step ks, element e (0..7) of the residual
// score products stands for. Code words are unpacked to match it: element 2i
// comes from field 4(g&1) + i of word 2ks + (g>>1) (INT2) and element 2i+1
// from the field 8 positions later.
__host__ __device__ constexpr int rs_coord(int ks, int g, int e) {
  return 32 * ks + 16 * (g >> 1) + 4 * (g & 1) + (e >> 1) + 8 * (e & 1);
}

// y = fp32(x / sqrt(D)) as an fp16 pair hi + lo: hi = fp16(y), lo = fp16(y - hi)
// (y - hi is exact in fp32), so hi + lo carries y to about 2^-23 relative. The
// residual scores run two fp16 products, one per part: one fp16 operand alone
// (2^-12 relative) moved heavy-tailed rows with residuals as large as the
// reference past 2e-3 in a CPU emulation of the kernel's roundings.
// The product is rounded to fp32 as written: the code generator fuses a
// product and its fp16 conversion into one mixed-precision fma (a single
// rounding) at some sites and not at others, and two kernels computing the
// same operand could then disagree by one fp16 ulp. The empty asm statement
// hands the conversions a finished fp32 value.
template <int D>
__device__ __forceinline__ void scaled_f16_pair(float x, _Float16& hi, _Float16& lo) {
  float y = x * RsqrtD<D>::v;
  asm volatile("" : "+v"(y));
  hi = (_Float16)y;
  lo = (_Float16)(y - (float)hi);
}

// One 8-coordinate operand chunk of the rotated query (x[p][i]: coordinate
// base + i + 8p) as fp16 hi and lo words in MFMA operand order; returns the
// chunk's sum of hi + lo. The prep kernel and the partial kernel's own
// rotation share this, so both give identical operands and offsets.
template <int D>
__device__ __forceinline__ float rotated_chunk(const float (&x)[2][4], uint4& hi, uint4& lo) {
  uint32_t wh[4], wl[4];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    _Float16 h0, l0, h1, l1;
    scaled_f16_pair<D>(x[0][i], h0, l0);
    scaled_f16_pair<D>(x[1][i], h1, l1);
    wh[i] = __builtin_bit_cast(uint32_t, f16x2_t{h0, h1});
    wl[i] = __builtin_bit_cast(uint32_t, f16x2_t{l0, l1});
    sum += ((float)h0 + (float)l0) + ((float)h1 + (float)l1);
  }
  hi = make_uint4(wh[0], wh[1], wh[2], wh[3]);
  lo = make_uint4(wl[0], wl[1], wl[2], wl[3]);
  return sum;
}

// Four lanes per query row (loop, b, hq), sixteen rows per wave. Lane g of a
// row loads the query in residual-score operand order: coordinates
// rs_coord(ks, g, 2i + p) = base + i + 8p (base = 32 ks + 16 (g >> 1) + 4 (g & 1))
// as x[ks][p][i]. The normalised Walsh-Hadamard transform runs over coordinate
// bits 0, 1, 3 and the k-step bits in registers and over bits 2 and 4 (lane
// bits 0 and 1) by DPP quad permutes. The record holds the fp16 hi parts of
// the rotated values in operand order (16 bytes per (ks, g)), the fp16 lo
// parts in the same order, and
// qoff[ks] = -(2^b + 2^(b-1) - 1/2) * (sum of the group's hi + lo values).
template <int D>
__global__ __launch_bounds__(64) void rq_query_prep(QueryPrepArgs a) {
  constexpr int NG = D / 32;
  const int lane = threadIdx.x;
  const int g = lane & 3;
  const int64_t row = (int64_t)blockIdx.x * 16 + (lane >> 2);
  const bool active = row < a.n_rows;
  const int64_t rr = active ? row : 0;
  const int loop = (int)(rr / ((int64_t)a.batch * a.n_q_heads));
  const int bits = a.bits[loop];
  const uint16_t* qr = a.q + rr * D + 16 * (g >> 1) + 4 * (g & 1);
  float x[NG][2][4];
#pragma unroll
  for (int ks = 0; ks < NG; ++ks)
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const uint2 u = *reinterpret_cast<const uint2*>(qr + 32 * ks + 8 * pp);
      x[ks][pp][0] = bf16_lo(u.x);
      x[ks][pp][1] = bf16_hi(u.x);
      x[ks][pp][2] = bf16_lo(u.y);
      x[ks][pp][3] = bf16_hi(u.y);
    }
#pragma unroll
  for (int ks = 0; ks < NG; ++ks) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int st = 1; st < 4; st <<= 1)  // coordinate bits 0 and 1
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!(i & st)) {
            const float u = x[ks][pp][i], w = x[ks][pp][i | st];
            x[ks][pp][i] = u + w;
            x[ks][pp][i | st] = u - w;
          }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // coordinate bit 3
      const float u = x[ks][0][i], w = x[ks][1][i];
      x[ks][0][i] = u + w;
      x[ks][1][i] = u - w;
    }
  }
#pragma unroll
  for (int st = 1; st < NG; st <<= 1)  // coordinate bits 5 (and 6)
#pragma unroll
    for (int ks = 0; ks < NG; ++ks)
      if (!(ks & st))
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float u = x[ks][pp][i], w = x[ks | st][pp][i];
            x[ks][pp][i] = u + w;
            x[ks | st][pp][i] = u - w;
          }
  // coordinate bit 2 (lane bit 0), then bit 4 (lane bit 1): the lower lane
  // keeps own + partner, the upper lane partner - own
  const float s1 = (g & 1) ? -1.0f : 1.0f, s2 = (g & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int ks = 0; ks < NG; ++ks)
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[ks][pp][i] = fmaf(s1, x[ks][pp][i], quad_xor<1>(x[ks][pp][i]));
#pragma unroll
  for (int ks = 0; ks < NG; ++ks)
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[ks][pp][i] = fmaf(s2, x[ks][pp][i], quad_xor<2>(x[ks][pp][i]));
  const float off = bits > 0 ? (float)(1 << bits) + (float)(1 << (bits - 1)) - 0.5f : 0.0f;
  unsigned char* rec = a.out + rr * MfmaGeom<D>::PREP_BYTES;
  float qo = 0.0f;
#pragma unroll
  for (int ks = 0; ks < NG; ++ks) {
    uint4 hi, lo;
    float sum = rotated_chunk<D>(x[ks], hi, lo);
    sum += quad_xor<1>(sum);
    sum += quad_xor<2>(sum);
    if (ks % 4 == g) qo = -off * sum;
    if (active) {
      *reinterpret_cast<uint4*>(rec + 16 * (4 * ks + g)) = hi;
      *reinterpret_cast<uint4*>(rec + 2 * D + 16 * (4 * ks + g)) = lo;
    }
  }
  if (active && g < NG) reinterpret_cast<float*>(rec + 4 * D)[g] = qo;
}

// ---------------------------------------------------------------------------
// partial kernel
// ---------------------------------------------------------------------------

// The lo parts of the rotated query (the B operands of the second residual
// score product), by where they live:
//  * kLoRegs: in registers (one 16-row block without INT3 / INT8 loops);
//  * kLoPads: INT3 / INT8 at one 16-row block. Those kernels are at their
//    register limit, so the block copies the lo parts from the prepared
//    records into the unused 128-byte pads that follow each 1 KB instruction
//    of the V tile (row r of the 16 in wave r / 4's pads, D / 64 pads a row);
//  * kLoRecord: 32-row blocks, and INT3 / INT8 in paired launches, read them
//    from the record at each use (at most 32 rows' records per block, so
//    these reads hit in the caches).
enum LoPlace { kLoRegs, kLoPads, kLoRecord };
template <int NB, bool WIDE, int SETS>
constexpr LoPlace kLoPlace = NB == 2 || (WIDE && SETS == 2) ? kLoRecord : (WIDE ? kLoPads : kLoRegs);

template <int D, int NB, LoPlace P>
struct QueryLo;
template <int D, int NB>
struct QueryLo<D, NB, kLoRegs> {
  uint4 v[NB][D / 32];
  __device__ __forceinline__ uint4 get(int nb, int ks, int) const { return v[nb][ks]; }
};
template <int D, int NB>
struct QueryLo<D, NB, kLoPads> {
  const unsigned char* row;  // this lane's row: its first pad
  // byte o of the row's 2D bytes sits in pad o / 128 at offset o % 128
  __device__ __forceinline__ uint4 get(int, int ks, int g) const {
    const int o = 16 * (4 * ks + g);
    return *reinterpret_cast<const uint4*>(row + (o >> 7) * MfmaGeom<D>::VT_STRIDE + (o & 127));
  }
  // LDS address of byte 0 of row r's lo parts (the pads of wave r / 4)
  static __device__ __forceinline__ unsigned char* row_of(unsigned char* smem, int wave_bytes, int r) {
    return smem + (r >> 2) * wave_bytes + (r & 3) * (D / 64) * MfmaGeom<D>::VT_STRIDE + 1024;
  }
};
template <int D, int NB>
struct QueryLo<D, NB, kLoRecord> {
  const unsigned char* rec[NB];  // the row's lo parts: 16 bytes per operand chunk (ks, g)
  __device__ __forceinline__ uint4 get(int nb, int ks, int g) const {
    return *reinterpret_cast<const uint4*>(rec[nb] + 16 * (4 * ks + g));
  }
};

// Issue the DMA of one residual loop's tile data (codes and scales of K and V).
template <int D, int BITS, bool FULL, bool SWZ>
__device__ __forceinline__ void stage_loop(const DecodeArgs& a, int li, unsigned char* base, int64_t row_base,
                                           int t0, int tlast, int lane) {
  constexpr int NG = D / 32;
  constexpr int W = D * BITS / 32;  // code words per vector
  unsigned char* kc_l = base;
  unsigned char* ks_l = kc_l + 128 * W;
  unsigned char* vc_l = ks_l + 64 * NG;
  unsigned char* vs_l = vc_l + 128 * W;
  const SlotPtrs sp = a.slot[li];
  if constexpr (FULL) {
    // All 32 tokens lie inside the sequence: buffer loads with the row as the
    // resource, the tile start as the scalar offset and per-lane constants.
    const uint32_t S = (uint32_t)a.seq_len;
    const auto kc_r = row_rsrc(sp.kc + row_base * W, S * 4u * W);
    const auto vc_r = row_rsrc(sp.vc + row_base * W, S * 4u * W);
    const auto ks_r = row_rsrc(sp.ks + row_base * NG, S * 2u * NG);
    const auto vs_r = row_rsrc(sp.vs + row_base * NG, S * 2u * NG);
    const uint32_t tc = (uint32_t)t0 * 4u * W, ts = (uint32_t)t0 * 2u * NG;
    const uint32_t kc_lane = 16u * (uint32_t)(lane ^ ((lane >> 4) & kKcSwz<D, BITS, SWZ>));
#pragma unroll
    for (int i = 0; i * 64 < 8 * W; ++i) {
      if (8 * W >= 64 * (i + 1) || 64 * i + lane < 8 * W) bdma16(kc_r, kc_lane, tc + 1024 * i, kc_l + 1024 * i);
    }
    if (16 * NG >= 64 || lane < 16 * NG) {
      bdma4(ks_r, 4u * (uint32_t)lane, ts, ks_l);
      bdma4(vs_r, 4u * (uint32_t)lane, ts, vs_l);
    }
    const uint32_t vc_lane = (uint32_t)(lane & 31) * (4u * W) + 4u * (uint32_t)(lane >> 5);
#pragma unroll
    for (int i = 0; i < W / 2; ++i) bdma4(vc_r, vc_lane, tc + 8 * i, vc_l + 256 * i);
    return;
  }
  if constexpr (W % 4 == 0) {
    // K code words in 16-byte chunks: chunk c -> token c / (W/4), words 4 (c % (W/4))
#pragma unroll
    for (int i = 0; i * 64 < 8 * W; ++i) {
      const int c = 64 * i + lane;
      if (8 * W >= 64 * (i + 1) || c < 8 * W) {
        const int tok = c / (W / 4), q4 = (c % (W / 4)) ^ ((c >> 4) & kKcSwz<D, BITS, SWZ>);
        dma16(sp.kc + (row_base + min(t0 + tok, tlast)) * W + 4 * q4, kc_l + 1024 * i);
      }
    }
  } else {
    // (INT3 at D = 64: 6 words per token) one word per lane: word idx -> token idx / W
#pragma unroll
    for (int i = 0; i * 64 < 32 * W; ++i) {
      const int idx = 64 * i + lane;
      if (32 * W >= 64 * (i + 1) || idx < 32 * W) {
        const int tok = idx / W, wd = idx % W;
        dma4(sp.kc + (row_base + min(t0 + tok, tlast)) * W + wd, kc_l + 256 * i);
      }
    }
  }
  // scales, 4 bytes per lane: lane -> token lane / (NG/2), pair lane % (NG/2)
  if (16 * NG >= 64 || lane < 16 * NG) {
    const int tok = lane / (NG / 2), pr = lane % (NG / 2);
    const int64_t vec = row_base + min(t0 + tok, tlast);
    dma4(sp.ks + vec * NG + 2 * pr, ks_l);
    dma4(sp.vs + vec * NG + 2 * pr, vs_l);
  }
  // V code words transposed: slot idx -> word idx / 32 of token idx % 32
#pragma unroll
  for (int i = 0; i < W / 2; ++i) {
    const int idx = 64 * i + lane;
    dma4(sp.vc + (row_base + min(t0 + (idx & 31), tlast)) * W + (idx >> 5), vc_l + 256 * i);
  }
}

// Constants kept in vector registers, so that mask-and-insert steps compile to
// one v_and_or_b32 (a gfx9 VOP3 instruction takes no literal operand).
struct Consts {
  uint32_t m2;    // 0x03000300: INT2 field at bits 8-9 of each half
  uint32_t m4;    // 0x03C003C0: INT4 field at bits 6-9 of each half
  uint32_t one;   // 0x3C003C00: fp16 1.0 in both halves
  uint32_t sel0;  // 0x000C000C: v_perm "zero byte" in bytes 0 and 2
  uint32_t m3lo;  // 0x01800180: INT3 low bits at bits 7-8 of each half
  uint32_t m3hi;  // 0x02000200: INT3 bit 2 at bit 9 of each half
  uint32_t m3s;   // 0x04000400: INT3 bit 2 at bit 2 of table-index bytes 1 and 3
};
template <bool WIDE>
__device__ __forceinline__ Consts make_consts() {
  Consts c{0x03000300u, 0x03C003C0u, 0x3C003C00u, 0x000C000Cu, 0x01800180u, 0x02000200u, 0x04000400u};
  if constexpr (!WIDE) {
    asm volatile("" : "+v"(c.m2), "+v"(c.m4), "+v"(c.one), "+v"(c.sel0));
  } else {
    // the masks in scalar registers (one per v_and_or_b32 fits the constant
    // bus), the or-operands in vector registers: the INT3 / INT8 kernels are
    // at their register limit
    asm volatile("" : "+s"(c.m2), "+s"(c.m4), "+v"(c.one), "+v"(c.sel0));
    asm volatile("" : "+s"(c.m3lo), "+s"(c.m3hi), "+s"(c.m3s));
  }
  return c;
}
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) { return (x & m) | o; }

// Residual scores of loop li added to this lane's score fragment. Rows of
// other loops get zero factors (qm = qo = 0), so every lane runs the same code.
template <int D, int NB, int BITS, bool SWZ, class QL>
__device__ __forceinline__ void residual_scores(const DecodeArgs& a, int li, const unsigned char* base,
                                                const uint4 (&qtB)[NB][D / 32], const QL& qtL,
                                                const float (&qoff)[NB][D / 32], const float (&qmul)[NB],
                                                const int (&my_loop)[NB], f32x4_t (&sc)[2][NB], int m, int g,
                                                const Consts& k) {
  constexpr int NG = D / 32;
  constexpr int W = D * BITS / 32;
  const unsigned char* kc_l = base;
  const unsigned char* ks_l = kc_l + 128 * W;
  const int G = a.group;
  float qm[NB], qo[NB][NG];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const bool mine = my_loop[nb] == li;
    qm[nb] = mine ? qmul[nb] : 0.0f;
#pragma unroll
    for (int ks = 0; ks < NG; ++ks) qo[nb][ks] = mine ? qoff[nb][ks] : 0.0f;
  }
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    // code words of token 16bk + m (this lane's A-operand row)
    const unsigned char* cw = kc_l + (16 * bk + m) * W * 4;
    const int kcr = (((16 * bk + m) * (W / 4)) >> 4) & kKcSwz<D, BITS, SWZ>;  // this token's chunk rotation
    uint4 kx[NG];
    if constexpr (BITS == 2) {
      // element 2i <- field 4(g&1) + i of word 2ks + (g>>1), element 2i+1 <- the field 8 later
      uint32_t wsel[NG];
      const bool hi = (g >> 1) != 0;
      const uint4 w0 = *reinterpret_cast<const uint4*>(cw + 16 * (0 ^ kcr));
      wsel[0] = hi ? w0.y : w0.x;
      wsel[1] = hi ? w0.w : w0.z;
      if constexpr (NG == 4) {
        const uint4 w1 = *reinterpret_cast<const uint4*>(cw + 16 * (1 ^ kcr));
        wsel[2] = hi ? w1.y : w1.x;
        wsel[3] = hi ? w1.w : w1.z;
      }
      const uint32_t pre = (g & 1) ? 0u : 8u;
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) {
        const uint32_t w = wsel[ks] << pre;
        kx[ks].x = and_or(w, k.m2, k.one);
        kx[ks].y = and_or(w >> 2, k.m2, k.one);
        kx[ks].z = and_or(w >> 4, k.m2, k.one);
        kx[ks].w = and_or(w >> 6, k.m2, k.one);
      }
    } else if constexpr (BITS == 8) {
      // element 2i <- byte i of word 8ks + 4(g>>1) + (g&1), element 2i+1 <- byte i of the word
      // two later. One v_perm puts both bytes at bytes 0 and 2; shifted up by 2 and or-ed into
      // 1.0 they give the fp16 values 1 + c/256.
      const uint32_t* row = reinterpret_cast<const uint32_t*>(cw);
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) {
        const int cb = 4 * ((2 * ks + (g >> 1)) ^ kcr) + (g & 1);  // the word's rotated place
        const uint32_t wa = row[cb];
        const uint32_t wb = row[cb + 2];
        kx[ks].x = (vperm(wb, wa, 0x0C040C00u) << 2) | k.one;
        kx[ks].y = (vperm(wb, wa, 0x0C050C01u) << 2) | k.one;
        kx[ks].z = (vperm(wb, wa, 0x0C060C02u) << 2) | k.one;
        kx[ks].w = (vperm(wb, wa, 0x0C070C03u) << 2) | k.one;
      }
    } else if constexpr (BITS == 3) {
      // The low two bits as in INT2 (plane words 2ks + (g>>1)), one bit lower: bits 7-8. Bit 2
      // comes from byte 2(g>>1) (element 2i) and byte 2(g>>1)+1 (element 2i+1) of the group's
      // bit-plane word, bit 4(g&1) + i of each, moved to bit 9. The fp16 values are 1 + c/8.
      const uint32_t* row = reinterpret_cast<const uint32_t*>(cw);
      const uint32_t pre = (g & 1) ? 0u : 8u;
      const uint32_t hsel = (uint32_t)(2 * (g >> 1)) | 0x0C000C00u | ((uint32_t)(2 * (g >> 1) + 1) << 16);
      const uint32_t hsh = 9u - 4u * (uint32_t)(g & 1);
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) {
        const uint32_t w = row[2 * ks + (g >> 1)] << pre;
        const uint32_t hb = row[D / 16 + ks];
        const uint32_t t = vperm(hb, hb, hsel) << hsh;
        kx[ks].x = and_or(t, k.m3hi, and_or(w >> 1, k.m3lo, k.one));
        kx[ks].y = and_or(t >> 1, k.m3hi, and_or(w >> 3, k.m3lo, k.one));
        kx[ks].z = and_or(t >> 2, k.m3hi, and_or(w >> 5, k.m3lo, k.one));
        kx[ks].w = and_or(t >> 3, k.m3hi, and_or(w >> 7, k.m3lo, k.one));
      }
    } else {
      // element 2i <- nibble 4(g&1) + i of word 4ks + 2(g>>1), element 2i+1 <- same nibble of
      // the next word. One v_perm puts the byte holding nibbles (i, i+1) of both words at
      // bytes 1 and 3; a shift then aligns either nibble at bits 6-9 of each half.
      const uint32_t b0 = 2u * (uint32_t)(g & 1);
      const uint32_t selA = ((b0) << 8) | ((4u + b0) << 24);
      const uint32_t selB = ((b0 + 1u) << 8) | ((5u + b0) << 24);
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) {
        const uint2 w = *reinterpret_cast<const uint2*>(cw + 16 * (ks ^ kcr) + 8 * (g >> 1));
        const uint32_t tA = vperm(w.y, w.x, selA), tB = vperm(w.y, w.x, selB);
        kx[ks].x = and_or(tA >> 2, k.m4, k.one);
        kx[ks].y = and_or(tA >> 6, k.m4, k.one);
        kx[ks].z = and_or(tB >> 2, k.m4, k.one);
        kx[ks].w = and_or(tB >> 6, k.m4, k.one);
      }
    }
    // k scales of this lane's four C-layout tokens 16bk + 4g + i
    uint32_t sw[4][(NG + 1) / 2];
    const unsigned char* sp = ks_l + (16 * bk + 4 * g) * NG * 2;
    if constexpr (NG == 4) {
      const uint4 u0 = *reinterpret_cast<const uint4*>(sp);
      const uint4 u1 = *reinterpret_cast<const uint4*>(sp + 16);
      sw[0][0] = u0.x; sw[0][1] = u0.y; sw[1][0] = u0.z; sw[1][1] = u0.w;
      sw[2][0] = u1.x; sw[2][1] = u1.y; sw[3][0] = u1.z; sw[3][1] = u1.w;
    } else {
      const uint4 u0 = *reinterpret_cast<const uint4*>(sp);
      sw[0][0] = u0.x; sw[1][0] = u0.y; sw[2][0] = u0.z; sw[3][0] = u0.w;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (li * G >= 16 * nb + 16 || li * G + G <= 16 * nb) continue;  // no row of loop li here
      // all group products first, so the MFMAs issue back to back: the hi
      // parts of the rotated query, then the lo parts into the same sums
      f32x4_t c[NG];
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) c[ks] = mma_f16(kx[ks], qtB[nb][ks], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) c[ks] = mma_f16(kx[ks], qtL.get(nb, ks, g), c[ks]);
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float s = (ks & 1) ? half_hi(sw[i][ks >> 1]) : half_lo(sw[i][ks >> 1]);
          sc[bk][nb][i] = fmaf(s, fmaf(c[ks][i], qm[nb], qo[nb][ks]), sc[bk][nb][i]);
        }
      }
    }
  }
}

// Residual PV of loop li into the shared residual accumulator.
template <int D, int NB, int BITS>
__device__ __forceinline__ void residual_pv(const DecodeArgs& a, int li, const unsigned char* base,
                                            const float (&p)[NB][8], const int (&my_loop)[NB],
                                            f32x4_t (&o_res)[NB][kResBlocks<D, NB>], int m, int g, const Consts& k) {
  constexpr int NG = D / 32;
  constexpr int W = D * BITS / 32;
  // INT2 / INT4 at NB = 1: codes decoded through the fp16 mantissa (see the
  // correction after the token loop); other widths through byte tables
  constexpr bool kMant = (BITS == 2 || BITS == 4) && NB == 1;
  const unsigned char* vc_l = base + 128 * W + 64 * NG;
  const unsigned char* vs_l = vc_l + 128 * W;
  const int G = a.group;
  // v scales of this lane's eight B-operand tokens (two runs of four)
  uint32_t vsw[8][(NG + 1) / 2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const unsigned char* sp = vs_l + (16 * h2 + 4 * g) * NG * 2;
    if constexpr (NG == 4) {
      const uint4 u0 = *reinterpret_cast<const uint4*>(sp);
      const uint4 u1 = *reinterpret_cast<const uint4*>(sp + 16);
      vsw[4 * h2 + 0][0] = u0.x; vsw[4 * h2 + 0][1] = u0.y;
      vsw[4 * h2 + 1][0] = u0.z; vsw[4 * h2 + 1][1] = u0.w;
      vsw[4 * h2 + 2][0] = u1.x; vsw[4 * h2 + 2][1] = u1.y;
      vsw[4 * h2 + 3][0] = u1.z; vsw[4 * h2 + 3][1] = u1.w;
    } else {
      const uint4 u0 = *reinterpret_cast<const uint4*>(sp);
      vsw[4 * h2 + 0][0] = u0.x; vsw[4 * h2 + 1][0] = u0.y;
      vsw[4 * h2 + 2][0] = u0.z; vsw[4 * h2 + 3][0] = u0.w;
    }
  }
  // A rows: coordinate 32grp + 16hf + m. Its code sits in byte `cb` of word
  // wv (INT2 and the INT3 low plane: byte m/4 of word 2grp + hf; INT4: byte
  // (m%8)/2 of word 4grp + 2hf + m/8; INT8: byte m%4 of word 8grp + 4hf +
  // m/4), `sh` bits up.
  uint32_t selx;
  uint32_t sh;
  if constexpr (BITS == 2 || BITS == 3) {
    selx = ((uint32_t)(m >> 2) << 8) | ((uint32_t)(4 + (m >> 2)) << 24);
    sh = 2u * (uint32_t)(m & 3);
  } else if constexpr (BITS == 8) {
    selx = (uint32_t)(m & 3) | 0x0C000C00u | ((uint32_t)(4 + (m & 3)) << 16);  // bytes 0 and 2
    sh = 0u;
  } else {
    const int f = m & 7;
    selx = ((uint32_t)(f >> 1) << 8) | ((uint32_t)(4 + (f >> 1)) << 24);
    sh = 4u * (uint32_t)(f & 1);
  }
  // INT3 bit 2 of coordinate 16hf + m: byte 2hf + m/8 of the bit-plane word, moved to bit 10
  const uint32_t hsh = 10u - (uint32_t)(m & 7);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (li * G >= 16 * nb + 16 || li * G + G <= 16 * nb) continue;
    // INT8 levels enter doubled (2c - 255), so P carries the factor 1/2
    const float mem = my_loop[nb] == li ? (BITS == 8 ? 0.5f : 1.0f) : 0.0f;
    float pm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pm[j] = p[nb][j] * mem;
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      // B operand: P s of the lane's eight tokens for this scale group (the
      // group's scale is half grp & 1 of word grp / 2)
      const bool hs = (grp & 1) != 0;
      uint4 bop;
      bop.x = mix_pair(pm[0], vsw[0][grp >> 1], pm[1], vsw[1][grp >> 1], hs);
      bop.y = mix_pair(pm[2], vsw[2][grp >> 1], pm[3], vsw[3][grp >> 1], hs);
      bop.z = mix_pair(pm[4], vsw[4][grp >> 1], pm[5], vsw[5][grp >> 1], hs);
      bop.w = mix_pair(pm[6], vsw[6][grp >> 1], pm[7], vsw[7][grp >> 1], hs);
      if constexpr (kMant) {
        // the group's weight sum (P s summed over the tile's tokens), in every
        // element of the block: an A operand of fp16 ones
        const uint4 ones = make_uint4(k.one, k.one, k.one, k.one);
        o_res[nb][2 * NG + grp] = mma_f16(ones, bop, o_res[nb][2 * NG + grp]);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if constexpr (BITS == 8) {
          const int wv = 8 * grp + 4 * hf + (m >> 2);
          const uint4 wa = *reinterpret_cast<const uint4*>(vc_l + (wv * 32 + 4 * g) * 4);
          const uint4 wb = *reinterpret_cast<const uint4*>(vc_l + (wv * 32 + 16 + 4 * g) * 4);
          // fp16 (1024 + 2c) - 1279 = 2c - 255, exact
          const f16x2_t off = {(_Float16)-1279.0f, (_Float16)-1279.0f};
          uint4 a8;
          a8.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, (vperm(wa.y, wa.x, selx) << 1) | 0x64006400u) + off);
          a8.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, (vperm(wa.w, wa.z, selx) << 1) | 0x64006400u) + off);
          a8.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, (vperm(wb.y, wb.x, selx) << 1) | 0x64006400u) + off);
          a8.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, (vperm(wb.w, wb.z, selx) << 1) | 0x64006400u) + off);
          o_res[nb][2 * grp + hf] = mma_f16(a8, bop, o_res[nb][2 * grp + hf]);
          continue;
        }
        const int wv = (BITS == 2 || BITS == 3) ? 2 * grp + hf : 4 * grp + 2 * hf + (m >> 3);
        const uint4 wa = *reinterpret_cast<const uint4*>(vc_l + (wv * 32 + 4 * g) * 4);
        const uint4 wb = *reinterpret_cast<const uint4*>(vc_l + (wv * 32 + 16 + 4 * g) * 4);
        // bytes 1 and 3 of y = the code bytes of two tokens, code at bits 8.. and 24..
        const uint32_t y0 = vperm(wa.y, wa.x, selx) >> sh;
        const uint32_t y1 = vperm(wa.w, wa.z, selx) >> sh;
        const uint32_t y2 = vperm(wb.y, wb.x, selx) >> sh;
        const uint32_t y3 = vperm(wb.w, wb.z, selx) >> sh;
        uint4 alo;
        if constexpr (BITS == 3) {
          // table index c = low bits | bit 2 << 2 in bytes 1 and 3
          const int wh = D / 16 + grp;
          const uint4 ha = *reinterpret_cast<const uint4*>(vc_l + (wh * 32 + 4 * g) * 4);
          const uint4 hb = *reinterpret_cast<const uint4*>(vc_l + (wh * 32 + 16 + 4 * g) * 4);
          const uint32_t hsel = (uint32_t)(2 * hf + (m >> 3)) | 0x0C000C00u | ((uint32_t)(4 + 2 * hf + (m >> 3)) << 16);
          alo.x = vperm(kLutInt3Hi, kLutInt3Lo, and_or(vperm(ha.y, ha.x, hsel) << hsh, k.m3s, and_or(y0, k.m2, k.sel0)));
          alo.y = vperm(kLutInt3Hi, kLutInt3Lo, and_or(vperm(ha.w, ha.z, hsel) << hsh, k.m3s, and_or(y1, k.m2, k.sel0)));
          alo.z = vperm(kLutInt3Hi, kLutInt3Lo, and_or(vperm(hb.y, hb.x, hsel) << hsh, k.m3s, and_or(y2, k.m2, k.sel0)));
          alo.w = vperm(kLutInt3Hi, kLutInt3Lo, and_or(vperm(hb.w, hb.z, hsel) << hsh, k.m3s, and_or(y3, k.m2, k.sel0)));
        } else if constexpr (kMant && BITS == 2) {
          // the code in the top mantissa bits of 1.0: fp16 1 + c/4
          alo.x = and_or(y0, k.m2, k.one);
          alo.y = and_or(y1, k.m2, k.one);
          alo.z = and_or(y2, k.m2, k.one);
          alo.w = and_or(y3, k.m2, k.one);
        } else if constexpr (kMant) {
          // the nibble at mantissa bits 6..9: fp16 1 + c/16
          alo.x = and_or(y0 >> 2, k.m4, k.one);
          alo.y = and_or(y1 >> 2, k.m4, k.one);
          alo.z = and_or(y2 >> 2, k.m4, k.one);
          alo.w = and_or(y3 >> 2, k.m4, k.one);
        } else {
          alo.x = vperm(0u, kLutInt2, and_or(y0, k.m2, k.sel0));
          alo.y = vperm(0u, kLutInt2, and_or(y1, k.m2, k.sel0));
          alo.z = vperm(0u, kLutInt2, and_or(y2, k.m2, k.sel0));
          alo.w = vperm(0u, kLutInt2, and_or(y3, k.m2, k.sel0));
        }
        o_res[nb][2 * grp + hf] = mma_f16(alo, bop, o_res[nb][2 * grp + hf]);
        if constexpr (BITS == 4 && !kMant) {
          uint4 ahi;
          ahi.x = vperm(0u, kLutInt4Hi, and_or(y0 >> 2, k.m2, k.sel0));
          ahi.y = vperm(0u, kLutInt4Hi, and_or(y1 >> 2, k.m2, k.sel0));
          ahi.z = vperm(0u, kLutInt4Hi, and_or(y2 >> 2, k.m2, k.sel0));
          ahi.w = vperm(0u, kLutInt4Hi, and_or(y3 >> 2, k.m2, k.sel0));
          o_res[nb][2 * grp + hf] = mma_f16(ahi, bop, o_res[nb][2 * grp + hf]);
        }
      }
    }
  }
}

// Issue every load of one tile: the residual loops' codes and scales and the
// V reference tile by LDS DMA into `buf`, the K reference into registers.
// WITH_K: the K reference into registers; WITH_V: the V tile into LDS.
template <int D, bool RESID, bool WIDE, bool FULL, bool WITH_K = true, bool WITH_V = true, bool SWZ8 = true>
__device__ __forceinline__ void issue_tile(const DecodeArgs& a, unsigned char* buf, const uint16_t* kbase,
                                           const uint16_t* vbase, int64_t row_base, int t0, int tlast, int lane,
                                           int m, int g, uint4 (&ka)[2][D / 32]) {
  using Gm = MfmaGeom<D>;
  constexpr int NG = Gm::NG;
  if constexpr (RESID) {
    // INT4 slots first, then INT2 (the launcher orders them): no branch per loop
    if constexpr (WIDE) {
      // slots INT8, INT4, INT3, INT2
      const int e8 = a.n8, e4 = e8 + a.n4, e3 = e4 + a.n3, e2 = e3 + a.n2;
      for (int li = 0; li < e8; ++li)
        stage_loop<D, 8, FULL, SWZ8>(a, li, buf + slot_lds_offset<D, true>(a, li), row_base, t0, tlast, lane);
      for (int li = e8; li < e4; ++li)
        stage_loop<D, 4, FULL, false>(a, li, buf + slot_lds_offset<D, true>(a, li), row_base, t0, tlast, lane);
      for (int li = e4; li < e3; ++li)
        stage_loop<D, 3, FULL, false>(a, li, buf + slot_lds_offset<D, true>(a, li), row_base, t0, tlast, lane);
      for (int li = e3; li < e2; ++li)
        stage_loop<D, 2, FULL, false>(a, li, buf + slot_lds_offset<D, true>(a, li), row_base, t0, tlast, lane);
    } else {
      for (int li = 0; li < a.n4; ++li)
        stage_loop<D, 4, FULL, true>(a, li, buf + slot_lds_offset<D, false>(a, li), row_base, t0, tlast, lane);
      for (int li = a.n4; li < a.n4 + a.n2; ++li)
        stage_loop<D, 2, FULL, true>(a, li, buf + slot_lds_offset<D, false>(a, li), row_base, t0, tlast, lane);
    }
  }
  if constexpr (FULL) {
    // the tile's 32 vectors are contiguous: 2D bytes each, one 16-byte chunk per lane
    const uint32_t rb = (uint32_t)a.seq_len * 2u * D;
    const uint32_t tb = (uint32_t)t0 * 2u * D;
    const uint32_t lane16 = 16u * (uint32_t)lane;
    if constexpr (WITH_V) {
      const auto v_r = row_rsrc(vbase, rb);
#pragma unroll
      for (int i = 0; i < Gm::VT_INSTR; ++i) bdma16(v_r, lane16, tb + 1024 * i, buf + i * Gm::VT_STRIDE);
    }
    if constexpr (WITH_K) {
      const auto k_r = row_rsrc(kbase, rb);
      const uint32_t koff = 2u * (uint32_t)(m * D + 8 * g);
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int ks = 0; ks < NG; ++ks) ka[bk][ks] = bload16(k_r, koff, tb + 32 * D * bk + 64 * ks);
    }
    return;
  }
  if constexpr (WITH_V) {
#pragma unroll
    for (int i = 0; i < Gm::VT_INSTR; ++i) {
      const int tok = i * Gm::VT_TOK + lane / (D / 8);
      dma16(vbase + (int64_t)min(t0 + tok, tlast) * D + 8 * (lane % (D / 8)), buf + i * Gm::VT_STRIDE);
    }
  }
  if constexpr (WITH_K) {
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      const uint16_t* kp = kbase + (int64_t)min(t0 + 16 * bk + m, tlast) * D + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) ka[bk][ks] = *reinterpret_cast<const uint4*>(kp + 32 * ks);
    }
  }
}

// Paged cache: whether the table entry of the tile at token t is a valid block
// (a tile without one takes no weight).
template <bool PAGED>
__device__ __forceinline__ bool tile_valid(const DecodeArgs& a, int b, int t) {
  if constexpr (PAGED) {
    const int blk = a.block_table[(int64_t)b * a.max_blocks + (t >> a.log2_block)];
    return blk >= 0 && blk < a.n_blocks;
  } else {
    return true;
  }
}

// Issue the tile at token t of sequence b, kv head kvh (blockIdx.y = z), dense
// or paged. Unclamped loads only when every token of the tile is one of this
// call's positions: positions past a sequence's length may hold any bits.
template <int D, bool RESID, bool WIDE, bool PAGED, bool SWZ8 = true>
__device__ __forceinline__ void issue_at(const DecodeArgs& a, unsigned char* buf, const uint16_t* kbase,
                                         const uint16_t* vbase, int64_t row_base, int b, int kvh, int z, int t,
                                         int t_end, int lane, int m, int g, uint4 (&ka)[2][D / 32]) {
  const bool full = t + kTile <= t_end;
  const int tlast = t_end - 1;
  if constexpr (PAGED) {
    const int blk = a.block_table[(int64_t)b * a.max_blocks + (t >> a.log2_block)];
    // vector index of token t; the tile's tokens follow it
    const int64_t tv = (((int64_t)blk * a.n_kv_heads + kvh) << a.log2_block) + (t & ((1 << a.log2_block) - 1));
    const uint16_t* kt = a.k[z] + tv * D;
    const uint16_t* vt = a.v[z] + tv * D;
    if (full) issue_tile<D, RESID, WIDE, true, true, true, SWZ8>(a, buf, kt, vt, tv, 0, tlast - t, lane, m, g, ka);
    else issue_tile<D, RESID, WIDE, false, true, true, SWZ8>(a, buf, kt, vt, tv, 0, tlast - t, lane, m, g, ka);
  } else {
    if (full) issue_tile<D, RESID, WIDE, true, true, true, SWZ8>(a, buf, kbase, vbase, row_base, t, tlast, lane, m, g, ka);
    else issue_tile<D, RESID, WIDE, false, true, true, SWZ8>(a, buf, kbase, vbase, row_base, t, tlast, lane, m, g, ka);
  }
}

// Paired launches: the two waves of a block share each tile's reference. The
// K tile goes to LDS (ahead of the V tile) in MFMA operand order: the
// instruction for k-step (bk, ks) has lane l = 16 g + m fetch the 16 bytes
// of token 16 bk + m at coordinate 32 ks + 8 g, so each wave later reads its
// A operand at lane * 16 of that instruction's 1 KB (no bank conflicts).
// Those instructions read half of each 128-byte line, so they keep the default
// cache policy. Wave 0 issues the K tile and its set's residual loops, wave 1
// the V tile and its set's.
template <int D>
constexpr int kPairKBytes = 2 * (D / 32) * 1024;

template <int D, bool RESID, bool WIDE, bool FULL>
__device__ __forceinline__ void pair_issue_tile(const DecodeArgs& a, unsigned char* smem, unsigned char* buf,
                                                const uint16_t* kbase, const uint16_t* vbase, int64_t row_base,
                                                int t0, int tlast, int lane, int m, int g, int wave) {
  using Gm = MfmaGeom<D>;
  constexpr int NG = Gm::NG;
  uint4 no_k[2][NG];  // issue_tile's K registers, not loaded here
  if (wave == 1) {
    // this set's residual loops and the V tile
    issue_tile<D, RESID, WIDE, FULL, false, true>(a, buf, kbase, vbase, row_base, t0, tlast, lane, m, g, no_k);
    return;
  }
  // wave 0: this set's residual loops, then the K tile in operand order
  issue_tile<D, RESID, WIDE, FULL, false, false>(a, buf, kbase, vbase, row_base, t0, tlast, lane, m, g, no_k);
  if constexpr (FULL) {
    const auto k_r = row_rsrc(kbase, (uint32_t)a.seq_len * 2u * D);
    const uint32_t voff = (uint32_t)(m * 2 * D + 16 * g);
    const uint32_t tb = (uint32_t)t0 * 2u * D;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) bdma16_keep(k_r, voff, tb + 32 * D * bk + 64 * ks, smem + (NG * bk + ks) * 1024);
  } else {
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      const uint16_t* kp = kbase + (int64_t)min(t0 + 16 * bk + m, tlast) * D + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) dma16_keep(kp + 32 * ks, smem + (NG * bk + ks) * 1024);
    }
  }
}

template <int D, bool RESID, bool WIDE, bool PAGED>
__device__ __forceinline__ void pair_issue_at(const DecodeArgs& a, unsigned char* smem, unsigned char* buf,
                                              const uint16_t* kbase, const uint16_t* vbase, int64_t row_base, int b,
                                              int kvh, int z, int t, int t_end, int lane, int m, int g, int wave) {
  const bool full = t + kTile <= t_end;
  const int tlast = t_end - 1;
  if constexpr (PAGED) {
    const int blk = a.block_table[(int64_t)b * a.max_blocks + (t >> a.log2_block)];
    const int64_t tv = (((int64_t)blk * a.n_kv_heads + kvh) << a.log2_block) + (t & ((1 << a.log2_block) - 1));
    const uint16_t* kt = a.k[z] + tv * D;
    const uint16_t* vt = a.v[z] + tv * D;
    if (full) pair_issue_tile<D, RESID, WIDE, true>(a, smem, buf, kt, vt, tv, 0, tlast - t, lane, m, g, wave);
    else pair_issue_tile<D, RESID, WIDE, false>(a, smem, buf, kt, vt, tv, 0, tlast - t, lane, m, g, wave);
  } else {
    if (full) pair_issue_tile<D, RESID, WIDE, true>(a, smem, buf, kbase, vbase, row_base, t, tlast, lane, m, g, wave);
    else pair_issue_tile<D, RESID, WIDE, false>(a, smem, buf, kbase, vbase, row_base, t, tlast, lane, m, g, wave);
  }
}

// Scores, online softmax and PV of one staged tile.
template <int D, int NB, bool RESID, bool WIDE, class QL>
__device__ __forceinline__ void compute_tile(const DecodeArgs& a, const unsigned char* buf, int t0, int t_end,
                                             int m, int g, const uint4 (&ka)[2][D / 32], const uint4 (&qB)[NB][D / 32],
                                             const uint4 (&qtB)[NB][D / 32], const QL& qtL,
                                             const float (&qoff)[NB][D / 32],
                                             const float (&qmul)[NB], const int (&my_loop)[NB],
                                             f32x4_t (&o_ref)[NB][D / 64][4], f32x4_t (&o_res)[NB][kResBlocks<D, NB>],
                                             float (&m_run)[NB], float (&l_run)[NB], const Consts& k) {
  using Gm = MfmaGeom<D>;
  constexpr int NG = Gm::NG, NH = Gm::NH;
  // ---- scores S^T[token][row]: lane holds tokens t0 + 16bk + 4g + i of row 16nb + m
  f32x4_t sc[2][NB];
#pragma unroll
  for (int bk = 0; bk < 2; ++bk)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) acc = mma_bf16(ka[bk][ks], qB[nb][ks], acc);
      sc[bk][nb] = acc;
    }
  if constexpr (RESID) {
    if constexpr (WIDE) {
      const int e8 = a.n8, e4 = e8 + a.n4, e3 = e4 + a.n3, e2 = e3 + a.n2;
      for (int li = 0; li < e8; ++li)
        residual_scores<D, NB, 8, NB == 1>(a, li, buf + slot_lds_offset<D, true>(a, li), qtB, qtL, qoff, qmul, my_loop, sc, m, g, k);
      for (int li = e8; li < e4; ++li)
        residual_scores<D, NB, 4, false>(a, li, buf + slot_lds_offset<D, true>(a, li), qtB, qtL, qoff, qmul, my_loop, sc, m, g, k);
      for (int li = e4; li < e3; ++li)
        residual_scores<D, NB, 3, false>(a, li, buf + slot_lds_offset<D, true>(a, li), qtB, qtL, qoff, qmul, my_loop, sc, m, g, k);
      for (int li = e3; li < e2; ++li)
        residual_scores<D, NB, 2, false>(a, li, buf + slot_lds_offset<D, true>(a, li), qtB, qtL, qoff, qmul, my_loop, sc, m, g, k);
    } else {
      for (int li = 0; li < a.n4; ++li)
        residual_scores<D, NB, 4, true>(a, li, buf + slot_lds_offset<D, false>(a, li), qtB, qtL, qoff, qmul, my_loop, sc, m, g, k);
      for (int li = a.n4; li < a.n4 + a.n2; ++li)
        residual_scores<D, NB, 2, true>(a, li, buf + slot_lds_offset<D, false>(a, li), qtB, qtL, qoff, qmul, my_loop, sc, m, g, k);
    }
  }

  // ---- online softmax (log2 domain); row statistics live in the row's 4 lanes
  float p[NB][8];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float zz[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) zz[j] = sc[j >> 2][nb][j & 3] * a.scale_log2;
    if (t0 + 2 * kTile16 > t_end) {  // tail tile: tokens past the split end take no weight
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (t0 + 16 * (j >> 2) + 4 * g + (j & 3) >= t_end) zz[j] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, zz[j]);
    mx = max_xor16_32(mx);
    const float m_new = fmaxf(m_run[nb], mx);
    const float alpha = fast_exp2(m_run[nb] - m_new);
    m_run[nb] = m_new;
    float ls = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[nb][j] = fast_exp2(zz[j] - m_new);
      ls += p[nb][j];
    }
    l_run[nb] = fmaf(l_run[nb], alpha, ls);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {  // running max moved for some row
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int r = 0; r < 4; ++r) o_ref[nb][hh][r] *= alpha;
      if constexpr (RESID) {
#pragma unroll
        for (int k = 0; k < kResBlocks<D, NB>; ++k) o_res[nb][k] *= alpha;
      }
    }
  }

  // ---- reference PV: O_ref^T[d][row] += V^T P^T, P = hi + lo in bf16
  uint4 pbh[NB], pbl[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u0 = __float_as_uint(p[nb][2 * i]), u1 = __float_as_uint(p[nb][2 * i + 1]);
      hi[i] = vperm(u1, u0, 0x07060302u);
      const float r0 = p[nb][2 * i] - __uint_as_float(u0 & 0xFFFF0000u);
      const float r1 = p[nb][2 * i + 1] - __uint_as_float(u1 & 0xFFFF0000u);
      lo[i] = vperm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
    }
    pbh[nb] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    pbl[nb] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    uint2 vv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = 16 * (j >> 2) + 4 * g + (j & 3);
      vv[j] = *reinterpret_cast<const uint2*>(buf + Gm::vt_offset(tok) + 2 * (64 * hh + 4 * m));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;
      uint4 av;
      av.x = vperm(r < 2 ? vv[1].x : vv[1].y, r < 2 ? vv[0].x : vv[0].y, sel);
      av.y = vperm(r < 2 ? vv[3].x : vv[3].y, r < 2 ? vv[2].x : vv[2].y, sel);
      av.z = vperm(r < 2 ? vv[5].x : vv[5].y, r < 2 ? vv[4].x : vv[4].y, sel);
      av.w = vperm(r < 2 ? vv[7].x : vv[7].y, r < 2 ? vv[6].x : vv[6].y, sel);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        o_ref[nb][hh][r] = mma_bf16(av, pbh[nb], o_ref[nb][hh][r]);
        o_ref[nb][hh][r] = mma_bf16(av, pbl[nb], o_ref[nb][hh][r]);
      }
    }
  }

  // ---- residual PV
  if constexpr (RESID) {
    if constexpr (WIDE) {
      const int e8 = a.n8, e4 = e8 + a.n4, e3 = e4 + a.n3, e2 = e3 + a.n2;
      for (int li = 0; li < e8; ++li)
        residual_pv<D, NB, 8>(a, li, buf + slot_lds_offset<D, true>(a, li), p, my_loop, o_res, m, g, k);
      for (int li = e8; li < e4; ++li)
        residual_pv<D, NB, 4>(a, li, buf + slot_lds_offset<D, true>(a, li), p, my_loop, o_res, m, g, k);
      for (int li = e4; li < e3; ++li)
        residual_pv<D, NB, 3>(a, li, buf + slot_lds_offset<D, true>(a, li), p, my_loop, o_res, m, g, k);
      for (int li = e3; li < e2; ++li)
        residual_pv<D, NB, 2>(a, li, buf + slot_lds_offset<D, true>(a, li), p, my_loop, o_res, m, g, k);
    } else {
      for (int li = 0; li < a.n4; ++li)
        residual_pv<D, NB, 4>(a, li, buf + slot_lds_offset<D, false>(a, li), p, my_loop, o_res, m, g, k);
      for (int li = a.n4; li < a.n4 + a.n2; ++li)
        residual_pv<D, NB, 2>(a, li, buf + slot_lds_offset<D, false>(a, li), p, my_loop, o_res, m, g, k);
    }
  }
}

// WIDE instantiations also take INT8 and INT3 loops; the others carry no code
// for them.
// Instantiations that can rotate the queries themselves (DecodeArgs::qprep
// NULL): one 16-row block of a residual launch over a dense cache with INT2 /
// INT4 loops.
// Where a partial block works: sequence b, kv head, split index and its
// position range [t_begin, t_end); n_b is sequence b's split count.
struct SplitPos {
  int b, kvh, split, t_begin, t_end, n_b;
};

__device__ __forceinline__ int units_of(int len, int S) {
  return (min(max(len, 0), S) + kDecodeTile - 1) / kDecodeTile;
}

// Blocks of a length-balanced plan with `per` units per split:
// Hkv * sum_b min(cap, max(1, ceil(u_b / per))), summed across the wave.
__device__ __forceinline__ long long balanced_blocks(const DecodeArgs& a, long long per, int lane) {
  const int B = a.batch, S = a.seq_len, cap = a.max_row_splits;
  long long n = 0;
  for (int i = lane; i < B; i += 64) n += min((long long)cap, max(1ll, (units_of(a.seq_lens[i], S) + per - 1) / per));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) n += __shfl_xor(n, o);
  return n * a.n_kv_heads;
}

// Length-balanced splits of a ragged decode (DecodeArgs::balance_target > 0).
// Sequence b holds u_b = ceil(min(len_b, S) / 64) units of 64 positions and
// gets n_b = min(max(1, ceil(u_b / per)), max_row_splits) splits of
// ceil(u_b / n_b) units each, so the blocks stream about the same number of
// positions whatever the lengths. `per` is the smallest unit count per split
// whose plan needs at most balance_target blocks (the launch's grid, all of it
// resident at once): found by bisection between ceil(U * Hkv / target) and
// ceil(U * Hkv / (target - B * Hkv)), U = sum_b u_b, since the block count
// falls as `per` grows and is at most U * Hkv / per + B * Hkv. Blocks
// enumerate (b, kv head, split) in that order; a block past the last returns
// false. The lengths are read 64 at a time and summed and scanned across the
// wave, so every wave of every block computes the same plan.
__device__ __forceinline__ bool balanced_split(const DecodeArgs& a, int work, int lane, SplitPos& sp) {
  const int B = a.batch, S = a.seq_len, H = a.n_kv_heads, cap = a.max_row_splits;
  const long long target = a.balance_target;
  long long u = 0;
  for (int i = lane; i < B; i += 64) u += units_of(a.seq_lens[i], S);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) u += __shfl_xor(u, o);
  const long long spread = max((long long)H, target - (long long)B * H);
  long long lo = max(1ll, (u * H + target - 1) / target), hi = max(lo, (u * H + spread - 1) / spread);
  while (lo < hi) {  // the smallest per in [lo, hi] whose plan fits the target
    const long long mid = (lo + hi) / 2;
    if (balanced_blocks(a, mid, lane) <= target) hi = mid;
    else lo = mid + 1;
  }
  const long long per = lo;
  long long base = 0;  // blocks of the sequences before this chunk
  for (int c = 0; c < B; c += 64) {
    const int i = c + lane;
    int ub = 0, nb = 0;
    if (i < B) {
      ub = units_of(a.seq_lens[i], S);
      nb = (int)min((long long)cap, max(1ll, (ub + per - 1) / per));
    }
    int incl = nb * H;  // inclusive scan of the blocks per sequence
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const long long chunk = __shfl(incl, 63);
    if (work < base + chunk) {
      const int excl = incl - nb * H;
      const bool mine = i < B && work >= base + excl && work < base + incl;
      const int src = __ffsll((long long)__ballot(mine)) - 1;
      const int n_b = __shfl(nb, src), u_b = __shfl(ub, src);
      const int local = work - (int)(base + __shfl(excl, src));
      const int len = min(max(a.seq_lens[c + src], 0), S);
      const int upb = (u_b + n_b - 1) / n_b;  // units per split
      sp.b = c + src;
      sp.kvh = local / n_b;
      sp.split = local % n_b;
      sp.n_b = n_b;
      sp.t_begin = sp.split * upb * kDecodeTile;
      sp.t_end = min(len, sp.t_begin + upb * kDecodeTile);
      return true;
    }
    base += chunk;
  }
  return false;
}

template <int NB, bool RESID, bool WIDE, bool PAGED, int SETS>
constexpr bool kRotatesQueries = NB == 1 && RESID && !WIDE && !PAGED && SETS == 1;

// The 16-row residual kernels have a second instantiation (VARW) whose blocks
// take their wave count from the launch (6 to kMaxWaves): INT8 loops, or
// several INT4 loops, stage so much per wave that two 4-wave blocks do not
// fit one CU's LDS, and one block of more waves keeps more tiles in flight
// than one of four. It reads prepared query records (no in-kernel rotation).
// 4-wave launches, and every other kernel, run the fixed four-wave code
// (measured 1.5-5% faster than the variable-wave code at four waves).
constexpr int kMaxWaves = 8;
template <int NB, bool RESID, bool WIDE, int SETS>
constexpr bool kVarWaves = NB == 1 && RESID && SETS == 1;

// SETS: the launch's argument sets (1 or 2). With one, a block is four
// waves (VARW: blockDim.x / 64) over one (batch, kv head, split), each
// taking every fourth (every blockDim.x / 64-th) tile. With
// two (paired launches), a block is two waves over one (batch, kv head,
// split): wave s computes set s's rows, both walk every tile of the split and
// share its reference K and V through LDS, each issuing half of the loads.
template <int D, int NB, bool RESID, bool WIDE, bool PAGED, int SETS, bool VARW>
__global__ __launch_bounds__((VARW ? 64 * kMaxWaves : 256))
__attribute__((amdgpu_waves_per_eu(RESID && NB == 2 ? 1 : 2,
                                                                     RESID && NB == 1 ? 2 : 4)))
void rq_decode_partial_mfma(DecodeLaunch launch) {
  using Gm = MfmaGeom<D>;
  constexpr int NG = Gm::NG, NH = Gm::NH;
  constexpr int NR = 16 * NB;
  constexpr int REC = 2 * D + 2;  // partial record: m, l, o_ref[D], o_res[D]
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: tile bases stay scalar
  static_assert(!VARW || kVarWaves<NB, RESID, WIDE, SETS>, "variable waves: the 16-row residual kernels only");
  constexpr bool VW = VARW;
  const int nw = VW ? __builtin_amdgcn_readfirstlane(blockDim.x >> 6) : 4;  // waves of a one-set block
  const int m = lane & 15, g = lane >> 4;
  constexpr bool PAIR = SETS == 2;
  const DecodeArgs& a = launch.set[PAIR ? wave : 0];
  const int work = blockIdx.x;
  const int z = blockIdx.y;
  const int S = a.seq_len;
  SplitPos sp;
  if (a.balance_target > 0) {
    // every wave of the block gets the same answer, so a surplus block exits whole
    if (!balanced_split(a, work, lane, sp)) return;
    if (a.row_splits != nullptr && sp.kvh == 0 && sp.split == 0 && threadIdx.x == 0) a.row_splits[sp.b] = sp.n_b;
  } else {
    sp.split = work % a.n_splits;
    const int bh0 = work / a.n_splits;
    sp.b = bh0 / a.n_kv_heads;
    sp.kvh = bh0 % a.n_kv_heads;
    sp.t_begin = sp.split * a.tokens_per_split;
    sp.t_end = min(S, sp.t_begin + a.tokens_per_split);
    if (a.seq_lens != nullptr) sp.t_end = min(sp.t_end, max(0, a.seq_lens[sp.b]));  // this sequence's prefix
  }
  const int split = __builtin_amdgcn_readfirstlane(sp.split);
  const int b = __builtin_amdgcn_readfirstlane(sp.b), kvh = __builtin_amdgcn_readfirstlane(sp.kvh);
  const int bh = b * a.n_kv_heads + kvh;
  const int G = a.group, R = a.n_rows;
  const int64_t row_base = (int64_t)bh * S;  // first cached vector of this (b, kv head)

  // ------------------------------------------------------------------ setup
  // B operands: bf16 Q^T for the reference scores (lane (m, g) holds
  // q[row 16nb+m][32ks + 8g .. +8]); fp16 rotated query + offsets (prepared).
  uint4 qB[NB][NG];
  uint4 qtB[NB][NG];
  constexpr LoPlace LP = kLoPlace<NB, WIDE, SETS>;
  QueryLo<D, NB, LP> qtL;
  float qoff[NB][NG];
  float qmul[NB];
  int my_loop[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = 16 * nb + m;
    my_loop[nb] = row < R ? row / G : -1;
    const int lb = my_loop[nb] >= 0 ? a.bits[my_loop[nb]] : 0;
    qmul[nb] = (float)(1 << lb);  // 2^b
    int64_t qrow = -1;
    if (row < R) qrow = ((int64_t)(a.loop_id[row / G] + z) * a.batch + b) * a.n_q_heads + kvh * G + row % G;
#pragma unroll
    for (int ks = 0; ks < NG; ++ks) {
      qB[nb][ks] = qrow >= 0 ? *reinterpret_cast<const uint4*>(a.q + qrow * D + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
      qtB[nb][ks] = make_uint4(0, 0, 0, 0);
      if constexpr (LP == kLoRegs) qtL.v[nb][ks] = make_uint4(0, 0, 0, 0);
      qoff[nb][ks] = 0.0f;
    }
    if constexpr (RESID && LP == kLoRecord) {
      // rows of other loops and padding rows read a real record too: their
      // residual score factors are zero, so only finiteness matters
      qtL.rec[nb] = a.qprep + (qrow >= 0 ? qrow : 0) * Gm::PREP_BYTES + 2 * D;
    }
    if constexpr (RESID) {
      if (qrow >= 0 && lb != 0 && a.qprep != nullptr) {
        const unsigned char* rec = a.qprep + qrow * Gm::PREP_BYTES;
#pragma unroll
        for (int ks = 0; ks < NG; ++ks) {
          qtB[nb][ks] = *reinterpret_cast<const uint4*>(rec + 16 * (4 * ks + g));
          if constexpr (LP == kLoRegs) qtL.v[nb][ks] = *reinterpret_cast<const uint4*>(rec + 2 * D + 16 * (4 * ks + g));
          qoff[nb][ks] = reinterpret_cast<const float*>(rec + 4 * D)[ks];
        }
      }
    }
  }

  // ------------------------------------------------------------ token loop
  // One tile buffer per wave: with two waves per SIMD, one wave's compute
  // covers the other's load latency. Measured on MI355X, a second buffer per
  // wave (prefetching the next tile) costs more occupancy than it hides.
  // Paired launches: the shared K tile first, then the shared V tile, then
  // each set's residual slots (lds_res_base)
  unsigned char* buf = PAIR ? smem + kPairKBytes<D> : smem + wave * a.lds_wave_bytes;
  if constexpr (RESID && LP == kLoPads) {
    // waves 0 .. 3 copy the lo parts of rows 4 wave .. 4 wave + 3 into their pads
    constexpr int kChunks = 2 * D / 16;  // 16-byte chunks per row
    const int r = 4 * wave + lane / kChunks, j = lane % kChunks;
    if (wave < 4 && lane < 4 * kChunks) {
      const int64_t qr = r < R ? ((int64_t)(a.loop_id[r / G] + z) * a.batch + b) * a.n_q_heads + kvh * G + r % G : 0;
      const uint4 v = *reinterpret_cast<const uint4*>(a.qprep + qr * Gm::PREP_BYTES + 2 * D + 16 * j);
      unsigned char* dst = QueryLo<D, NB, kLoPads>::row_of(smem, a.lds_wave_bytes, r);
      *reinterpret_cast<uint4*>(dst + (16 * j >> 7) * Gm::VT_STRIDE + (16 * j & 127)) = v;
    }
    qtL.row = QueryLo<D, NB, kLoPads>::row_of(smem, a.lds_wave_bytes, m);
    __syncthreads();
  }
  f32x4_t o_ref[NB][NH][4];
  f32x4_t o_res[NB][kResBlocks<D, NB>];
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.0f;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int r = 0; r < 4; ++r) o_ref[nb][hh][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kResBlocks<D, NB>; ++k) o_res[nb][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int t_begin = __builtin_amdgcn_readfirstlane(sp.t_begin);
  const int t_end = __builtin_amdgcn_readfirstlane(sp.t_end);
  const uint16_t* kbase = a.k[z] + row_base * D;
  const uint16_t* vbase = a.v[z] + row_base * D;
  const int kStep = PAIR ? kTile : nw * kTile;  // tokens between a wave's consecutive tiles

  const Consts kc = make_consts<WIDE>();
  uint4 ka[2][NG];
  int t0 = t_begin + (PAIR ? 0 : wave * kTile);
  // (only where the extra copy of the tile body adds no register spills)
  if constexpr (kRotatesQueries<NB, RESID, WIDE, PAGED, SETS> && !VARW) {
    if (a.qprep == nullptr) {
      // The residual-score operand is computed here rather than read from
      // prepared records: the block's 16 rows go 16 / NG to a wave, 4 NG lanes
      // per row with one 8-coordinate operand chunk (ks, g) each, and the
      // block shares them through LDS after the tiles. The query loads go out
      // with the wave's first tile.
      constexpr int kLanesRow = 4 * NG, kRowsWave = 64 / kLanesRow;
      constexpr int QS = 2 * D + 16;  // LDS bytes per row: operand chunks, then 4 NG offsets
      unsigned char* qreg = smem + 4 * a.lds_wave_bytes;
      const int rr = kRowsWave * wave + lane / kLanesRow;  // block row this lane rotates
      const int c = lane % kLanesRow, cks = c >> 2, cg = c & 3;
      const int lbr = rr < R ? a.bits[rr / G] : 0;
      int64_t qr = -1;
      if (rr < R && lbr != 0) qr = ((int64_t)(a.loop_id[rr / G] + z) * a.batch + b) * a.n_q_heads + kvh * G + rr % G;
      const uint16_t* qs = a.q + (qr >= 0 ? qr : 0) * D + 32 * cks + 16 * (cg >> 1) + 4 * (cg & 1);
      const uint2 q0 = qr >= 0 ? *reinterpret_cast<const uint2*>(qs) : make_uint2(0, 0);
      const uint2 q1 = qr >= 0 ? *reinterpret_cast<const uint2*>(qs + 8) : make_uint2(0, 0);
      if (t0 < t_end) issue_at<D, RESID, WIDE, PAGED, NB == 1>(a, buf, kbase, vbase, row_base, b, kvh, z, t0, t_end, lane, m, g, ka);
      wait_vmem();
      // x[p][i]: coordinate base + i + 8p. Butterflies on coordinate bits 0, 1
      // and 3 in the lane, then across the row's lanes: the k-step bits (lane
      // bits 2 and up), coordinate bit 2 (lane bit 0) and bit 4 (lane bit 1).
      // The lower lane keeps own + partner, the upper one partner - own. This
      // is the prep kernel's stage order, so both give identical values.
      float x[2][4] = {{bf16_lo(q0.x), bf16_hi(q0.x), bf16_lo(q0.y), bf16_hi(q0.y)},
                       {bf16_lo(q1.x), bf16_hi(q1.x), bf16_lo(q1.y), bf16_hi(q1.y)}};
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int st = 1; st < 4; st <<= 1)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!(i & st)) {
              const float u = x[pp][i], w = x[pp][i | st];
              x[pp][i] = u + w;
              x[pp][i | st] = u - w;
            }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float u = x[0][i], w = x[1][i];
        x[0][i] = u + w;
        x[1][i] = u - w;
      }
#pragma unroll
      for (int k = 2; k < 2 + NG / 2 + 2; ++k) {  // lane bits 2 (, 3), then 0 and 1
        const int st = 1 << (k < 2 + NG / 2 ? k : k - 2 - NG / 2);
        const float sg = (c & st) ? -1.0f : 1.0f;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[pp][i] = fmaf(sg, x[pp][i], __shfl_xor(x[pp][i], st));
      }
      uint4 w_hi, w_lo;
      float sum = rotated_chunk<D>(x, w_hi, w_lo);
      sum += quad_xor<1>(sum);  // the group's four chunks (same k-step)
      sum += quad_xor<2>(sum);
      // the hi parts and the offsets first, then the lo parts in the same slots
      if (rr < 16) {
        *reinterpret_cast<uint4*>(qreg + rr * QS + 16 * c) = w_hi;
        if (cg == 0) {
          const float off = lbr > 0 ? (float)(1 << lbr) + (float)(1 << (lbr - 1)) - 0.5f : 0.0f;
          *reinterpret_cast<float*>(qreg + rr * QS + 2 * D + 4 * cks) = -off * sum;
        }
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) {
        qtB[0][ks] = *reinterpret_cast<const uint4*>(qreg + m * QS + 16 * (4 * ks + g));
        qoff[0][ks] = *reinterpret_cast<const float*>(qreg + m * QS + 2 * D + 4 * ks);
      }
      __syncthreads();
      if (rr < 16) *reinterpret_cast<uint4*>(qreg + rr * QS + 16 * c) = w_lo;
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) qtL.v[0][ks] = *reinterpret_cast<const uint4*>(qreg + m * QS + 16 * (4 * ks + g));
      wave_sync_lds();
      // the first tile, already staged (its own copy of the tile body, so the
      // K registers are not live across the loop below)
      if (t0 < t_end) {
        compute_tile<D, NB, RESID, WIDE>(a, buf, t0, t_end, m, g, ka, qB, qtB, qtL, qoff, qmul, my_loop, o_ref, o_res, m_run,
                                         l_run, kc);
        wait_lds();
        wave_sync_lds();
        t0 += kStep;
      }
    }
  }
  if constexpr (PAIR) {
    // both waves walk every tile; each waits for its own loads, then the
    // barrier makes the other wave's half visible, and a second barrier
    // keeps the shared buffers until both have read them
    for (; t0 < t_end; t0 += kStep) {
      if (!tile_valid<PAGED>(a, b, t0)) continue;  // both waves see the same table entry
      pair_issue_at<D, RESID, WIDE, PAGED>(a, smem, buf, kbase, vbase, row_base, b, kvh, z, t0, t_end, lane, m, g,
                                           wave);
      wait_vmem();
      __syncthreads();
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int ks = 0; ks < NG; ++ks) ka[bk][ks] = *reinterpret_cast<const uint4*>(smem + (NG * bk + ks) * 1024 + 16 * lane);
      compute_tile<D, NB, RESID, WIDE>(a, buf, t0, t_end, m, g, ka, qB, qtB, qtL, qoff, qmul, my_loop, o_ref, o_res,
                                       m_run, l_run, kc);
      __syncthreads();
    }
  } else {
    for (; t0 < t_end; t0 += kStep) {
      if (!tile_valid<PAGED>(a, b, t0)) continue;  // no valid page: the tile takes no weight
      issue_at<D, RESID, WIDE, PAGED, NB == 1>(a, buf, kbase, vbase, row_base, b, kvh, z, t0, t_end, lane, m, g, ka);
      wait_vmem();
      wave_sync_lds();
      compute_tile<D, NB, RESID, WIDE>(a, buf, t0, t_end, m, g, ka, qB, qtB, qtL, qoff, qmul, my_loop, o_ref, o_res,
                                       m_run, l_run, kc);
      wait_lds();
      wave_sync_lds();  // the buffer is free for the next tile's DMA
    }
  }

  // At NB = 1 the INT2 / INT4 rows accumulated sum P s (1 + c/2^b). The level
  // c - (2^(b-1) - 1/2) is 2^b (1 + c/2^b) - (2^b + 2^(b-1) - 1/2), so the
  // level sum is 2^b times the accumulator minus that constant times the
  // group's weight sum. Rows of INT3 / INT8 loops hold level sums already.
  if constexpr (RESID && NB == 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int lb = my_loop[nb] >= 0 ? a.bits[my_loop[nb]] : 0;
      const bool mant = lb == 2 || lb == 4;
      const float mulc = mant ? qmul[nb] : 1.0f;
      const float offc = mant ? 1.5f * qmul[nb] - 0.5f : 0.0f;
#pragma unroll
      for (int k = 0; k < 2 * NG; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) o_res[nb][k][i] = fmaf(mulc, o_res[nb][k][i], -offc * o_res[nb][2 * NG + k / 2][i]);
    }
  }

  // ------------------------------------------------- merge the block's waves
  // Each wave leaves its record for every row, [m, l, o_ref[D], o_res[D]] (the
  // residual part only with residual loops), in its LDS slot. Then each wave
  // merges whole rows (rows wave, wave + nw, ...), its lanes across the record:
  // the slots are summed in wave order (reproducible), each scaled by
  // 2^(m_w - max m), and the result is the row's partial record. The merge
  // needs nw * NR * (2D + 2) floats of LDS. In a paired launch each wave holds
  // whole rows of its own set, and copies its slot out as the rows' records.
  constexpr int SREC = RESID ? 2 * D + 2 : D + 2;  // record floats this launch writes
  __syncthreads();
  float* slots = reinterpret_cast<float*>(smem);
  {
    float* slot = slots + wave * NR * SREC;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float* rs = slot + (16 * nb + m) * SREC;
      float ls = l_run[nb];
      ls += __shfl_xor(ls, 16);
      ls += __shfl_xor(ls, 32);
      if (g == 0) {
        rs[0] = m_run[nb];
        rs[1] = ls;
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) rs[2 + 64 * hh + 4 * (4 * g + i) + r] = o_ref[nb][hh][r][i];
      if constexpr (RESID) {
#pragma unroll
        for (int k = 0; k < 2 * NG; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) rs[2 + D + 16 * k + 4 * g + i] = o_res[nb][k][i];
      }
    }
  }
  __syncthreads();
  if constexpr (PAIR) {
    const float* slot = slots + wave * NR * SREC;
    for (int r = 0; r < R; ++r) {
      const int loop = a.loop_id[r / G] + z;
      const int hq = kvh * G + r % G;
      float* dst = a.ws + ((((int64_t)loop * a.batch + b) * a.n_q_heads + hq) * a.rec_splits + a.split_base + split) * REC;
#pragma unroll
      for (int j = 0; j * 64 < SREC; ++j) {
        const int e = lane + 64 * j;
        if (e < SREC) dst[e] = slot[r * SREC + e];
      }
    }
    return;
  }
  constexpr int MW = VW ? kMaxWaves : 4;
  for (int r = wave; r < R; r += nw) {
    const float* s0 = slots + r * SREC;
    float mw[MW], mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < MW; ++w) {
      mw[w] = w < nw ? s0[w * NR * SREC] : -INFINITY;
      mm = fmaxf(mm, mw[w]);
    }
    float fw[MW];
#pragma unroll
    for (int w = 0; w < MW; ++w) fw[w] = mw[w] == -INFINITY ? 0.0f : exp2f(mw[w] - mm);
    const int loop = a.loop_id[r / G] + z;
    const int hq = kvh * G + r % G;
    float* dst = a.ws + ((((int64_t)loop * a.batch + b) * a.n_q_heads + hq) * a.rec_splits + a.split_base + split) * REC;
#pragma unroll
    for (int j = 0; j * 64 < SREC; ++j) {
      const int e = lane + 64 * j;
      if (e < SREC) {
        float val = mm;
        if (e > 0) {
          val = 0.0f;
#pragma unroll
          for (int w = 0; w < MW; ++w)
            if (w < nw) val = fmaf(fw[w], s0[w * NR * SREC + e], val);
        }
        dst[e] = val;
      }
    }
  }
  // Without residual loops the record ends after o_ref, unless the call's
  // combine reads residual accumulators (other launches of the call carry
  // residual loops): then this launch's rows get a zero one.
  if constexpr (!RESID) {
    if (a.zero_residual) {
      for (int i = threadIdx.x; i < R * D; i += blockDim.x) {
        const int r = i / D, e = i % D;
        const int loop = a.loop_id[r / G] + z;
        const int hq = kvh * G + r % G;
        a.ws[((((int64_t)loop * a.batch + b) * a.n_q_heads + hq) * a.rec_splits + a.split_base + split) * REC + D + 2 + e] =
            0.0f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int decode_wave_lds_bytes(int head_dim, const int32_t* bits, int n_loops) {
  int bytes = head_dim == 128 ? MfmaGeom<128>::VT_BYTES : MfmaGeom<64>::VT_BYTES;
  for (int i = 0; i < n_loops; ++i) bytes += loop_lds_bytes(head_dim, bits[i]);
  return bytes;
}

int decode_loop_lds_bytes(int head_dim, int bits) { return loop_lds_bytes(head_dim, bits); }

int query_prep_bytes(int head_dim) {
  return head_dim == 128 ? MfmaGeom<128>::PREP_BYTES : MfmaGeom<64>::PREP_BYTES;
}

// LDS bytes of one block of nw waves: the larger of the merge slots and the
// wave tiles (rotate: plus the 16 rows' rotated-query operands after them)
static int block_lds_bytes(int d, int nb, int wave_bytes, bool residual, bool rotate, int nw = 4) {
  const int nr = 16 * nb;
  const int merge = nw * nr * (residual ? 2 * d + 2 : d + 2) * 4;  // every wave's records of every row
  const int tiles = nw * wave_bytes + (rotate ? 16 * (2 * d + 16) : 0);
  return merge > tiles ? merge : tiles;
}

// Waves per block of a one-set launch: four, except in the 16-row residual
// kernels when two 4-wave blocks overflow a CU's LDS: then as many as one
// block's LDS holds (at most kMaxWaves, two per SIMD), if that is six or
// more. The waves of a block take equal shares of its tiles; on MI355X five
// waves (one SIMD holding two) ran slower than four, while six and seven ran
// 15-28% faster on the mixed_s32k INT8 layers and about 20% faster with two
// or three INT4 loops.
static int block_waves(int d, int nb, int wave_bytes, bool residual) {
  if (!residual || nb != 1 || 2 * block_lds_bytes(d, nb, wave_bytes, true, false) <= kMaxBlockLds) return 4;
  int nw = 4;
  while (nw < kMaxWaves && block_lds_bytes(d, nb, wave_bytes, true, false, nw + 1) <= kMaxBlockLds) ++nw;
  return nw >= 6 ? nw : 4;
}

// LDS bytes of a paired block: the shared K and V tiles, both sets' residual
// slots, or (if larger) both waves' record slots for the final copy-out
static int pair_lds_bytes(int d, const DecodeArgs* sets, bool residual) {
  const int vt = d == 128 ? MfmaGeom<128>::VT_BYTES : MfmaGeom<64>::VT_BYTES;
  int tiles = (d == 128 ? kPairKBytes<128> : kPairKBytes<64>) + vt;
  for (int i = 0; i < 2; ++i) tiles += decode_wave_lds_bytes(d, sets[i].bits, residual ? sets[i].n_loops_launch : 0) - vt;
  const int merge = 2 * 16 * (residual ? 2 * d + 2 : d + 2) * 4;
  return merge > tiles ? merge : tiles;
}

int decode_launch_waves(const DecodeArgs* sets, int n_sets, int head_dim, bool residual) {
  if (n_sets == 2) return 2;
  if (sets[0].n_rows > 16) return 4;
  return block_waves(head_dim, 1, decode_wave_lds_bytes(head_dim, sets[0].bits, residual ? sets[0].n_loops_launch : 0),
                     residual);
}

int decode_launch_lds_bytes(const DecodeArgs* sets, int n_sets, int head_dim, bool residual, bool rotate) {
  if (n_sets == 2) return pair_lds_bytes(head_dim, sets, residual);
  int rows = 0, lds = 0;
  for (int i = 0; i < n_sets; ++i) rows = std::max(rows, sets[i].n_rows);
  const int nb = rows > 16 ? 2 : 1;
  for (int i = 0; i < n_sets; ++i) {
    const int wave = decode_wave_lds_bytes(head_dim, sets[i].bits, residual ? sets[i].n_loops_launch : 0);
    lds = std::max(lds, block_lds_bytes(head_dim, nb, wave, residual, rotate && residual && nb == 1));
  }
  return lds;
}

template <int D, int NB, bool RESID, bool WIDE, bool PAGED, int SETS, bool VARW = false>
static void launch_mfma_kernel(const DecodeLaunch& l, dim3 grid, int lds, int nw, hipStream_t stream) {
  // Lift the default dynamic-LDS cap once per instantiation and device (the
  // attribute belongs to the current device; devices past 63 set it every time).
  static std::atomic<uint64_t> lifted{0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t{1} << dev : 0;
  if ((lifted.load(std::memory_order_relaxed) & bit) == 0) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&rq_decode_partial_mfma<D, NB, RESID, WIDE, PAGED, SETS, VARW>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kMaxBlockLds);
    lifted.fetch_or(bit, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((rq_decode_partial_mfma<D, NB, RESID, WIDE, PAGED, SETS, VARW>), grid, dim3(64 * nw), lds, stream,
                     l);
}

template <int D, int NB, bool PAGED, int SETS>
static hipError_t launch_mfma_dp(const DecodeLaunch& l, dim3 grid, int lds, int nw, bool residual, bool wide,
                                 hipStream_t stream) {
  // waves per block: two in a paired launch, four in every one-set kernel
  // except the 16-row residual ones, which take 4 .. kMaxWaves
  const bool var = kVarWaves<NB, true, false, SETS> && residual;
  if (SETS == 2 ? nw != 2 : (var ? nw < 4 || nw > kMaxWaves : nw != 4)) return hipErrorInvalidValue;
  // a residual launch without prepared records must be a 4-wave one that
  // rotates the queries itself
  if (residual && l.set[0].qprep == nullptr &&
      (nw != 4 ||
       (wide ? !kRotatesQueries<NB, true, true, PAGED, SETS> : !kRotatesQueries<NB, true, false, PAGED, SETS>)))
    return hipErrorInvalidValue;
  if (!residual) {
    launch_mfma_kernel<D, NB, false, false, PAGED, SETS>(l, grid, lds, nw, stream);
    return hipSuccess;
  }
  if constexpr (kVarWaves<NB, true, false, SETS>) {
    if (nw != 4) {
      if (wide) launch_mfma_kernel<D, NB, true, true, PAGED, SETS, true>(l, grid, lds, nw, stream);
      else launch_mfma_kernel<D, NB, true, false, PAGED, SETS, true>(l, grid, lds, nw, stream);
      return hipSuccess;
    }
  }
  if (wide) launch_mfma_kernel<D, NB, true, true, PAGED, SETS>(l, grid, lds, nw, stream);
  else launch_mfma_kernel<D, NB, true, false, PAGED, SETS>(l, grid, lds, nw, stream);
  return hipSuccess;
}

template <int D, int NB>
static hipError_t launch_mfma_d(DecodeLaunch& l, dim3 grid, bool residual, hipStream_t stream) {
  bool wide = false;
  for (int i = 0; i < l.n_sets; ++i) {
    DecodeArgs& a = l.set[i];
    a.lds_wave_bytes = decode_wave_lds_bytes(D, a.bits, residual ? a.n_loops_launch : 0);
    wide = wide || a.n8 + a.n3 > 0;
  }
  const bool paged = l.set[0].block_table != nullptr;
  if (l.n_sets == 2) {  // two sets of at most 16 rows: one wave each, sharing the reference tiles
    l.set[0].lds_res_base = 0;
    l.set[1].lds_res_base = l.set[0].lds_wave_bytes - MfmaGeom<D>::VT_BYTES;
    const int lds = pair_lds_bytes(D, l.set, residual);
    if (paged) return launch_mfma_dp<D, 1, true, 2>(l, grid, lds, 2, residual, wide, stream);
    return launch_mfma_dp<D, 1, false, 2>(l, grid, lds, 2, residual, wide, stream);
  }
  const DecodeArgs& a = l.set[0];
  const int nw = block_waves(D, NB, a.lds_wave_bytes, residual);
  const int lds = block_lds_bytes(D, NB, a.lds_wave_bytes, residual, residual && NB == 1 && a.qprep == nullptr, nw);
  if (paged) return launch_mfma_dp<D, NB, true, 1>(l, grid, lds, nw, residual, wide, stream);
  return launch_mfma_dp<D, NB, false, 1>(l, grid, lds, nw, residual, wide, stream);
}

hipError_t launch_decode_partial(const DecodeArgs* sets, int n_sets, int head_dim, int n_z, bool residual,
                                 hipStream_t stream) {
  if (n_sets < 1 || n_sets > kMaxSets) return hipErrorInvalidValue;
  DecodeLaunch l{};
  l.n_sets = n_sets;
  int rows = 0;
  for (int i = 0; i < n_sets; ++i) {
    l.set[i] = sets[i];
    rows = std::max(rows, sets[i].n_rows);
  }
  const DecodeArgs& a = sets[0];
  const int64_t rows_kv = (int64_t)a.batch * a.n_kv_heads;
  const int64_t n_work =
      a.balance_target > 0 ? balanced_max_blocks(rows_kv, a.n_kv_heads, a.seq_len) : a.n_splits * rows_kv;
  const dim3 grid((unsigned)n_work, n_z);
  const bool two = rows > 16;
  hipError_t e;
  if (head_dim == 128) e = two ? launch_mfma_d<128, 2>(l, grid, residual, stream) : launch_mfma_d<128, 1>(l, grid, residual, stream);
  else e = two ? launch_mfma_d<64, 2>(l, grid, residual, stream) : launch_mfma_d<64, 1>(l, grid, residual, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_query_prep(const QueryPrepArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n_rows + 15) / 16));
  if (head_dim == 128) hipLaunchKernelGGL(rq_query_prep<128>, grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(rq_query_prep<64>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rq
