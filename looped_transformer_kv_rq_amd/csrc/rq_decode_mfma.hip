// Split-S decode attention over the ResidualQuant cache on gfx950 matrix cores.
//
// ResidualQuant (newx.sg page, Abstract): an earlier loop's K/V is the bf16
// final-loop reference plus a rotated INT2/INT4 residual with a least-squares
// fp16 scale per 32 coordinates. One call attends every loop's queries over
// the cache and streams the reference once for all of them. The rotation H
// (normalised Walsh-Hadamard) is symmetric, so
//   score  = q . k_ref + (H q) . (s * lev)
//   output = sum_t p_t v_ref,t + H sum_t p_t (s * lev)_t.
// Each query is rotated once. The residual terms stay in the rotated domain,
// and a split applies H to its residual accumulator a single time.
//
// One block is four independent waves over one split of one (batch, kv head)
// row. A wave takes 32-token tiles (tiles w, w+4, ...). Every query row of the
// kv head (all loops x the G query heads, at most 32 = two 16-row blocks) is
// one MFMA column. All products run on v_mfma_f32_16x16x32:
//  * reference scores S^T = K_ref Q^T (bf16; exact products, fp32 sums). The
//    K tile is loaded straight into the A operand with 16-byte loads;
//  * residual scores per loop and scale group (fp16). Codes become the fp16
//    value 1 + c / 2^b by masking them into the mantissa of 1.0 (one shift
//    and one and-or per two codes). The per-row constant of that offset is
//    taken out exactly afterwards: q.(c - o) = 2^b (q.val) - (2^b + o) sum(q);
//  * reference PV, O_ref^T += V^T P^T (bf16). P is split into bf16 hi + lo
//    halves (error ~2^-16), and V^T is read from a per-wave LDS tile;
//  * residual PV, O_res^T += lev^T (P s)^T (fp16). Levels decode exactly
//    through a v_perm byte lookup table (INT2: {-1.5,-0.5,0.5,1.5}; INT4 as
//    4 lev_hi + lev_lo, two table lookups). The rows of other loops carry
//    P s = 0, so every loop shares one accumulator.
// The MFMA output layout (lane l holds rows 4 (l / 16) + i of column l % 16)
// gives each lane one query row and four tokens per 16-token block. The
// online-softmax statistics of a row therefore stay within the row's four
// lanes, and the P fragment is already the B operand of the PV products.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ uint32_t pack_rtz(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}
__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr uint32_t kLutInt2 = 0x3E38B8BEu;    // fp16 high bytes of -1.5, -0.5, 0.5, 1.5
constexpr uint32_t kLutInt4Hi = 0x4640C0C6u;  // fp16 high bytes of -6, -2, 2, 6 (4 * INT2 level)
constexpr int kTile = 32;
constexpr int kCodeStride = 36;  // dwords per code-word row (32 tokens + pad) in LDS

template <int D>
struct MfmaGeom {
  static constexpr int NG = D / 32;    // scale groups = k-steps of the score products
  static constexpr int NH = D / 64;    // 64-coordinate halves of the reference PV
  static constexpr int VTS = D + 8;    // bf16 elements per V tile row in LDS
  static constexpr int VTILE_BYTES = kTile * VTS * 2;
};

// LDS bytes one wave needs during the token loop (V tile + one loop's code words)
__host__ __device__ constexpr int mfma_wave_lds_bytes(int d, int max_bits) {
  return kTile * (d + 8) * 2 + (d * max_bits / 32) * kCodeStride * 4;
}

template <int D, int NB, bool RESID>
__global__ __launch_bounds__(256) void rq_decode_partial_mfma(DecodeArgs a) {
  using Gm = MfmaGeom<D>;
  constexpr int NG = Gm::NG, NH = Gm::NH, VTS = Gm::VTS;
  constexpr int NR = 16 * NB;
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int split = blockIdx.x % a.n_splits;
  const int bh = blockIdx.x / a.n_splits;
  const int z = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int G = a.group, R = a.n_rows, S = a.seq_len;
  const int64_t row_base = (int64_t)bh * S;  // first cached vector of this (b, kv head)

  // ------------------------------------------------------------------ setup
  // Reference-score B operand (bf16 Q^T): lane (m, g) holds q[row 16nb+m][32ks + 8g .. +8].
  uint4 qB[NB][NG];
  int my_loop[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = 16 * nb + m;
    my_loop[nb] = row < R ? row / G : -1;
    const uint16_t* qp = nullptr;
    if (row < R) {
      const int loop = a.loop_base + row / G + z;
      qp = a.q + (((int64_t)loop * a.batch + b) * a.n_q_heads + kvh * G + row % G) * D;
    }
#pragma unroll
    for (int ks = 0; ks < NG; ++ks)
      qB[nb][ks] = qp ? *reinterpret_cast<const uint4*>(qp + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
  }

  // Residual-score B operand (fp16 rotated query). Lane (m, g), k-step ks,
  // element 2i <-> coordinate 32ks + 16(g>>1) + 4(g&1) + i, element 2i+1 <-> +8;
  // this matches how the code words are unpacked below.
  uint4 qtB[NB][NG];
  float qoff[NB][NG];   // -(2^b + offset) * sum of the group's rotated query coordinates
  float qmul[NB];       // 2^b of the row's own loop
  (void)qtB; (void)qoff; (void)qmul;
  if constexpr (RESID) {
    float* qs = reinterpret_cast<float*>(smem);  // [NR][D]
    for (int i = threadIdx.x; i < NR * D; i += 256) {
      const int r = i / D, d = i % D;
      float v = 0.0f;
      if (r < R) {
        const int loop = a.loop_base + r / G + z;
        const uint16_t qb = a.q[(((int64_t)loop * a.batch + b) * a.n_q_heads + kvh * G + r % G) * D + d];
        v = __uint_as_float((uint32_t)qb << 16);
      }
      qs[i] = v;
    }
    __syncthreads();
    for (int h = 1; h < D; h <<= 1) {
      for (int i = threadIdx.x; i < NR * D / 2; i += 256) {
        const int r = i / (D / 2), k = i % (D / 2);
        const int lo = r * D + (k / h) * 2 * h + (k % h);
        const float x = qs[lo], y = qs[lo + h];
        qs[lo] = x + y;
        qs[lo + h] = x - y;
      }
      __syncthreads();
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float* qr = qs + (16 * nb + m) * D;
      const int lb = my_loop[nb] >= 0 ? a.bits[my_loop[nb]] : 0;
      qmul[nb] = lb == 4 ? 16.0f : 4.0f;
      const float off = lb == 4 ? 23.5f : 5.5f;  // 2^b + (2^(b-1) - 1/2)
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) {
        uint32_t w[4];
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * ks + 16 * (g >> 1) + 4 * (g & 1) + i;
          const f16x2_t h2 = {(_Float16)(qr[d0] * RsqrtD<D>::v), (_Float16)(qr[d0 + 8] * RsqrtD<D>::v)};
          w[i] = __builtin_bit_cast(uint32_t, h2);
          part += (float)h2[0] + (float)h2[1];
        }
        qtB[nb][ks] = make_uint4(w[0], w[1], w[2], w[3]);
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        qoff[nb][ks] = -off * part;
      }
    }
    __syncthreads();  // the per-wave tile buffers below reuse this LDS
  }

  // ------------------------------------------------------------ token loop
  unsigned char* wbase = smem + wave * a.lds_wave_bytes;
  uint16_t* vt = reinterpret_cast<uint16_t*>(wbase);                        // [32][VTS] bf16
  uint32_t* ct = reinterpret_cast<uint32_t*>(wbase + Gm::VTILE_BYTES);     // [words][kCodeStride]

  f32x4_t o_ref[NB][NH][4];
  f32x4_t o_res[NB][2 * NG];
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
    for (int k = 0; k < 2 * NG; ++k) o_res[nb][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  (void)o_res;

  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(S, t_begin + a.tokens_per_split);
  const uint16_t* kbase = a.k[z] + row_base * D;
  const uint16_t* vbase = a.v[z] + row_base * D;

  for (int t0 = t_begin + wave * kTile; t0 < t_end; t0 += 4 * kTile) {
    // stage the V tile: 16-byte chunk c -> token c / (D/8), column 8 (c % (D/8))
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int c = lane + 64 * i;
      const int tok = c / (D / 8), col = c % (D / 8);
      const int t = min(t0 + tok, t_end - 1);
      const uint4 v = *reinterpret_cast<const uint4*>(vbase + (int64_t)t * D + 8 * col);
      *reinterpret_cast<uint4*>(vt + tok * VTS + 8 * col) = v;
    }

    // ---- scores S^T[token][row]: lane holds tokens t0 + 16bk + 4g + i of row 16nb + m
    f32x4_t sc[2][NB];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      const int t = min(t0 + 16 * bk + m, t_end - 1);
      const uint16_t* kp = kbase + (int64_t)t * D + 8 * g;
      uint4 ka[NG];
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) ka[ks] = *reinterpret_cast<const uint4*>(kp + 32 * ks);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NG; ++ks) acc = mma_bf16(ka[ks], qB[nb][ks], acc);
        sc[bk][nb] = acc;
      }
    }

    if constexpr (RESID) {
      for (int li = 0; li < a.n_loops_launch; ++li) {
        const int bits = a.bits[li];
        if (bits == 0) continue;
        const int words = D * bits / 32;
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
          // code words of token t0 + 16bk + m (this lane's A-operand row)
          const int ta = min(t0 + 16 * bk + m, t_end - 1);
          const uint32_t* cw = a.kc[li] + (row_base + ta) * words;
          uint4 kx[NG];
          if (bits == 2) {
            uint32_t wsel[NG];
            if constexpr (D == 128) {
              const uint4 w0 = *reinterpret_cast<const uint4*>(cw);
              const uint4 w1 = *reinterpret_cast<const uint4*>(cw + 4);
              const bool hi = (g >> 1) != 0;
              wsel[0] = hi ? w0.y : w0.x;
              wsel[1] = hi ? w0.w : w0.z;
              wsel[2] = hi ? w1.y : w1.x;
              wsel[3] = hi ? w1.w : w1.z;
            } else {
              const uint4 w0 = *reinterpret_cast<const uint4*>(cw);
              const bool hi = (g >> 1) != 0;
              wsel[0] = hi ? w0.y : w0.x;
              wsel[1] = hi ? w0.w : w0.z;
            }
            const uint32_t pre = (g & 1) ? 0u : 8u;
#pragma unroll
            for (int ks = 0; ks < NG; ++ks) {
              const uint32_t w = wsel[ks] << pre;
              kx[ks].x = (w & 0x03000300u) | 0x3C003C00u;
              kx[ks].y = ((w >> 2) & 0x03000300u) | 0x3C003C00u;
              kx[ks].z = ((w >> 4) & 0x03000300u) | 0x3C003C00u;
              kx[ks].w = ((w >> 6) & 0x03000300u) | 0x3C003C00u;
            }
          } else {
            const uint32_t f4 = 4u * (uint32_t)(4 * (g & 1));
#pragma unroll
            for (int ks = 0; ks < NG; ++ks) {
              const uint2 w = *reinterpret_cast<const uint2*>(cw + 4 * ks + 2 * (g >> 1));
              uint32_t e[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t c0 = __builtin_amdgcn_ubfe(w.x, f4 + 4 * i, 4);
                const uint32_t c1 = __builtin_amdgcn_ubfe(w.y, f4 + 4 * i, 4);
                e[i] = (c1 << 22) | (c0 << 6) | 0x3C003C00u;
              }
              kx[ks] = make_uint4(e[0], e[1], e[2], e[3]);
            }
          }
          // k scales of this lane's four C-layout tokens
          float ksc[4][NG];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tt = min(t0 + 16 * bk + 4 * g + i, t_end - 1);
            const uint16_t* sp = a.ks[li] + (row_base + tt) * NG;
            if constexpr (NG == 4) {
              const uint2 u = *reinterpret_cast<const uint2*>(sp);
              ksc[i][0] = half_lo(u.x); ksc[i][1] = half_hi(u.x);
              ksc[i][2] = half_lo(u.y); ksc[i][3] = half_hi(u.y);
            } else {
              const uint32_t u = *reinterpret_cast<const uint32_t*>(sp);
              ksc[i][0] = half_lo(u); ksc[i][1] = half_hi(u);
            }
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            if (li * G >= 16 * nb + 16 || li * G + G <= 16 * nb) continue;  // no row of loop li here
            f32x4_t r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NG; ++ks) {
              const f32x4_t c = mma_f16(kx[ks], qtB[nb][ks], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int i = 0; i < 4; ++i) r[i] = fmaf(ksc[i][ks], fmaf(c[i], qmul[nb], qoff[nb][ks]), r[i]);
            }
            if (my_loop[nb] == li) {
#pragma unroll
              for (int i = 0; i < 4; ++i) sc[bk][nb][i] += r[i];
            }
          }
        }
      }
    }

    // ---- online softmax (log2 domain); row statistics live in the row's 4 lanes
    float p[NB][8];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float zz[8];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = t0 + 16 * (j >> 2) + 4 * g + (j & 3);
        zz[j] = t < t_end ? sc[j >> 2][nb][j & 3] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, zz[j]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[nb], mx);
      const float alpha = exp2f(m_run[nb] - m_new);
      m_run[nb] = m_new;
      float ls = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[nb][j] = exp2f(zz[j] - m_new);
        ls += p[nb][j];
      }
      l_run[nb] = fmaf(l_run[nb], alpha, ls);
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int r = 0; r < 4; ++r) o_ref[nb][hh][r] *= alpha;
      if constexpr (RESID) {
#pragma unroll
        for (int k = 0; k < 2 * NG; ++k) o_res[nb][k] *= alpha;
      }
    }

    wave_sync_lds();  // V tile visible to the whole wave

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
        vv[j] = *reinterpret_cast<const uint2*>(vt + tok * VTS + 64 * hh + 4 * m);
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

    // ---- residual PV: O_res^T[d][row] += lev^T (P s)^T, per loop
    if constexpr (RESID) {
      for (int li = 0; li < a.n_loops_launch; ++li) {
        const int bits = a.bits[li];
        if (bits == 0) continue;
        const int words = D * bits / 32;
        // stage this tile's V code words transposed: ct[word][token]
        const int chunks = kTile * words / 4;
        for (int c = lane; c < chunks; c += 64) {
          const int tok = c / (words / 4), q4 = c % (words / 4);
          const int t = min(t0 + tok, t_end - 1);
          const uint4 w = *reinterpret_cast<const uint4*>(a.vc[li] + (row_base + t) * words + 4 * q4);
          ct[(4 * q4 + 0) * kCodeStride + tok] = w.x;
          ct[(4 * q4 + 1) * kCodeStride + tok] = w.y;
          ct[(4 * q4 + 2) * kCodeStride + tok] = w.z;
          ct[(4 * q4 + 3) * kCodeStride + tok] = w.w;
        }
        // v scales of this lane's eight B-operand tokens
        uint32_t vsw[8][(NG + 1) / 2];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tt = min(t0 + 16 * (j >> 2) + 4 * g + (j & 3), t_end - 1);
          const uint16_t* sp = a.vs[li] + (row_base + tt) * NG;
          if constexpr (NG == 4) {
            const uint2 u = *reinterpret_cast<const uint2*>(sp);
            vsw[j][0] = u.x;
            vsw[j][1] = u.y;
          } else {
            vsw[j][0] = *reinterpret_cast<const uint32_t*>(sp);
          }
        }
        wave_sync_lds();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if (li * G >= 16 * nb + 16 || li * G + G <= 16 * nb) continue;
          const float mem = my_loop[nb] == li ? 1.0f : 0.0f;
          float pm[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) pm[j] = p[nb][j] * mem;
#pragma unroll
          for (int grp = 0; grp < NG; ++grp) {
            uint32_t bw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t s0 = vsw[2 * i][grp >> 1], s1 = vsw[2 * i + 1][grp >> 1];
              const float f0 = (grp & 1) ? half_hi(s0) : half_lo(s0);
              const float f1 = (grp & 1) ? half_hi(s1) : half_lo(s1);
              bw[i] = pack_rtz(pm[2 * i] * f0, pm[2 * i + 1] * f1);
            }
            const uint4 bop = make_uint4(bw[0], bw[1], bw[2], bw[3]);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              // A rows: coordinate 32grp + 16hf + m; its code sits in word wv, field f
              int wv, sh;
              uint32_t selx;
              if (bits == 2) {
                wv = 2 * grp + hf;
                selx = ((uint32_t)(m >> 2) << 8) | ((uint32_t)(4 + (m >> 2)) << 24);
                sh = 2 * (m & 3);
              } else {
                wv = 4 * grp + 2 * hf + (m >> 3);
                const int f = m & 7;
                selx = ((uint32_t)(f >> 1) << 8) | ((uint32_t)(4 + (f >> 1)) << 24);
                sh = 4 * (f & 1);
              }
              const uint4 wa = *reinterpret_cast<const uint4*>(ct + wv * kCodeStride + 4 * g);
              const uint4 wb = *reinterpret_cast<const uint4*>(ct + wv * kCodeStride + 16 + 4 * g);
              const uint32_t cw[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
              uint32_t y[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) y[i] = vperm(cw[2 * i + 1], cw[2 * i], selx) >> sh;
              uint4 alo;
              alo.x = vperm(0u, kLutInt2, (y[0] & 0x03000300u) | 0x000C000Cu);
              alo.y = vperm(0u, kLutInt2, (y[1] & 0x03000300u) | 0x000C000Cu);
              alo.z = vperm(0u, kLutInt2, (y[2] & 0x03000300u) | 0x000C000Cu);
              alo.w = vperm(0u, kLutInt2, (y[3] & 0x03000300u) | 0x000C000Cu);
              o_res[nb][2 * grp + hf] = mma_f16(alo, bop, o_res[nb][2 * grp + hf]);
              if (bits == 4) {
                uint4 ahi;
                ahi.x = vperm(0u, kLutInt4Hi, ((y[0] >> 2) & 0x03000300u) | 0x000C000Cu);
                ahi.y = vperm(0u, kLutInt4Hi, ((y[1] >> 2) & 0x03000300u) | 0x000C000Cu);
                ahi.z = vperm(0u, kLutInt4Hi, ((y[2] >> 2) & 0x03000300u) | 0x000C000Cu);
                ahi.w = vperm(0u, kLutInt4Hi, ((y[3] >> 2) & 0x03000300u) | 0x000C000Cu);
                o_res[nb][2 * grp + hf] = mma_f16(ahi, bop, o_res[nb][2 * grp + hf]);
              }
            }
          }
        }
        wave_sync_lds();  // code tile free for the next loop
      }
    }
    wave_sync_lds();  // V tile free for the next tile
  }

  // ------------------------------------------------ merge the four waves
  __syncthreads();
  float* mw = reinterpret_cast<float*>(smem);  // [4][NR]
  float* lw = mw + 4 * NR;                     // [4][NR]
  float* acc_ref = lw + 4 * NR;                // [NR][D]
  float* acc_res = acc_ref + NR * D;           // [NR][D]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float ls = l_run[nb];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if (g == 0) {
      mw[wave * NR + 16 * nb + m] = m_run[nb];
      lw[wave * NR + 16 * nb + m] = ls;
    }
  }
  __syncthreads();
  float fw[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = 16 * nb + m;
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, mw[w * NR + row]);
    fw[nb] = m_run[nb] == -INFINITY ? 0.0f : exp2f(m_run[nb] - mm);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float* ar = acc_ref + (16 * nb + m) * D;
        float* as = acc_res + (16 * nb + m) * D;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int d = 64 * hh + 4 * (4 * g + i) + r;
              const float v = fw[nb] * o_ref[nb][hh][r][i];
              ar[d] = (w == 0) ? v : ar[d] + v;
            }
        if constexpr (RESID) {
#pragma unroll
          for (int k = 0; k < 2 * NG; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int d = 16 * k + 4 * g + i;  // k = 2 grp + hf -> 32 grp + 16 hf
              const float v = fw[nb] * o_res[nb][k][i];
              as[d] = (w == 0) ? v : as[d] + v;
            }
        }
      }
    }
    __syncthreads();
  }
  if constexpr (RESID) {
    for (int h = 1; h < D; h <<= 1) {
      for (int i = threadIdx.x; i < NR * D / 2; i += 256) {
        const int r = i / (D / 2), k = i % (D / 2);
        const int lo = r * D + (k / h) * 2 * h + (k % h);
        const float x = acc_res[lo], y = acc_res[lo + h];
        acc_res[lo] = x + y;
        acc_res[lo + h] = x - y;
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < R * (D + 2); i += 256) {
    const int r = i / (D + 2), e = i % (D + 2);
    const int loop = a.loop_base + r / G + z;
    const int hq = kvh * G + r % G;
    float* dst = a.ws + ((((int64_t)loop * a.batch + b) * a.n_q_heads + hq) * a.n_splits + split) * (D + 2);
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, mw[w * NR + r]);
    float val;
    if (e == 0) {
      val = mm;
    } else if (e == 1) {
      float ls = 0.0f;
      for (int w = 0; w < 4; ++w) ls += mw[w * NR + r] == -INFINITY ? 0.0f : exp2f(mw[w * NR + r] - mm) * lw[w * NR + r];
      val = ls;
    } else {
      const int d = e - 2;
      val = acc_ref[r * D + d] + (RESID ? acc_res[r * D + d] * RsqrtD<D>::v : 0.0f);
    }
    dst[e] = val;
  }
}

// LDS bytes of one block: the larger of the setup / merge area and 4 wave tiles
static int mfma_block_lds_bytes(int d, int nb, int max_bits) {
  const int nr = 16 * nb;
  const int merge = (8 * nr + 2 * nr * d) * 4;
  const int tiles = 4 * mfma_wave_lds_bytes(d, max_bits);
  return merge > tiles ? merge : tiles;
}

template <int D, int NB>
static void launch_mfma_d(DecodeArgs a, dim3 grid, bool residual, int max_bits, hipStream_t stream) {
  a.lds_wave_bytes = mfma_wave_lds_bytes(D, max_bits);
  const int lds = mfma_block_lds_bytes(D, NB, max_bits);
  if (residual) hipLaunchKernelGGL((rq_decode_partial_mfma<D, NB, true>), grid, dim3(256), lds, stream, a);
  else hipLaunchKernelGGL((rq_decode_partial_mfma<D, NB, false>), grid, dim3(256), lds, stream, a);
}

hipError_t launch_decode_partial(const DecodeArgs& a, int head_dim, int n_z, bool residual, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.n_splits * a.batch * a.n_kv_heads), n_z);
  int max_bits = 0;
  for (int li = 0; li < a.n_loops_launch; ++li) max_bits = a.bits[li] > max_bits ? a.bits[li] : max_bits;
  if (!residual) max_bits = 0;
  const bool two = a.n_rows > 16;
  if (head_dim == 128) {
    if (two) launch_mfma_d<128, 2>(a, grid, residual, max_bits, stream);
    else launch_mfma_d<128, 1>(a, grid, residual, max_bits, stream);
  } else {
    if (two) launch_mfma_d<64, 2>(a, grid, residual, max_bits, stream);
    else launch_mfma_d<64, 1>(a, grid, residual, max_bits, stream);
  }
  return hipGetLastError();
}

}  // namespace rq
