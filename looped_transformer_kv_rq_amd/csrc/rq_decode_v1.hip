// Split-S decode attention over the ResidualQuant cache: straightforward
// VALU form, and the log-sum-exp combine of the split partials.
//
// ResidualQuant (newx.sg page, Abstract): an earlier loop's K/V is the
// final-loop reference plus a rotated low-bit residual. Decode attention reads
// both and never materialises K/V. Because the Walsh-Hadamard matrix H is
// symmetric:
//   q . (k_ref + H (s * lev)) = q . k_ref + (H q) . (s * lev)
//   sum_t p_t (v_ref + H (s * lev))_t = sum_t p_t v_ref,t + H sum_t p_t (s * lev)_t
// So each query is rotated once, the residual scores are taken in the rotated
// domain, and a split applies one inverse rotation to its residual accumulator.
//
// Block = 4 waves, one (split, batch * kv head) pair per blockIdx.x, loop per blockIdx.y. Scores use one lane
// per token, and the PV step uses one lane per output coordinate. A block
// writes one partial (running max in log2 units, sum of weights, unnormalised
// output) per query row.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// all lanes of one wave see each other's LDS writes
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int BITS>
__device__ __forceinline__ float level_of(uint32_t word, int j) {
  constexpr float off = (float)(1 << (BITS - 1)) - 0.5f;
  return (float)((word >> (BITS * j)) & ((1u << BITS) - 1u)) - off;
}

__device__ __forceinline__ float level_any(const uint32_t* codes_vec, int d, int bits) {
  if (bits == 2) return level_of<2>(codes_vec[d >> 4], d & 15);
  return level_of<4>(codes_vec[d >> 3], d & 7);
}

template <int D, int NR, bool RESID>
__global__ __launch_bounds__(256) void rq_decode_partial_v1(DecodeArgs a) {
  constexpr int DJ = D / 64;
  constexpr int NG = D / 32;
  __shared__ float qs[NR][D];
  __shared__ float qt[RESID ? NR : 1][D];
  __shared__ float pb[4][NR][64];
  __shared__ float mw[4][NR];
  __shared__ float lw[4][NR];

  const int split = blockIdx.x % a.n_splits;
  const int bh = blockIdx.x / a.n_splits;
  const int z = blockIdx.y;
  const int b = bh / a.n_kv_heads;
  const int kvh = bh % a.n_kv_heads;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int G = a.group;
  const int R = a.n_rows;
  const int S = a.seq_len;

  // ---- queries (and their rotation) into LDS
  for (int i = threadIdx.x; i < NR * D; i += 256) {
    const int r = i / D, d = i % D;
    float val = 0.0f;
    if (r < R) {
      const int loop = a.loop_base + r / G + z;
      const int hq = kvh * G + r % G;
      const uint16_t qb = a.q[(((int64_t)loop * a.batch + b) * a.n_q_heads + hq) * D + d];
      val = __uint_as_float((uint32_t)qb << 16);
    }
    qs[r][d] = val;
    if constexpr (RESID) qt[r][d] = val;
  }
  __syncthreads();
  if constexpr (RESID) {
    // unnormalised transform of every query row; 1/sqrt(D) is applied with the scale
    for (int h = 1; h < D; h <<= 1) {
      for (int i = threadIdx.x; i < NR * D / 2; i += 256) {
        const int r = i / (D / 2), k = i % (D / 2);
        const int lo = (k / h) * 2 * h + (k % h);
        const float x = qt[r][lo], y = qt[r][lo + h];
        qt[r][lo] = x + y;
        qt[r][lo + h] = x - y;
      }
      __syncthreads();
    }
  }

  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(S, t_begin + a.tokens_per_split);
  const uint16_t* kbase = a.k[z] + (int64_t)bh * S * D;
  const uint16_t* vbase = a.v[z] + (int64_t)bh * S * D;

  float m[NR], l[NR], o_ref[NR][DJ], o_res[RESID ? NR : 1][DJ];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
      o_ref[r][j] = 0.0f;
      if constexpr (RESID) o_res[r][j] = 0.0f;
    }
  }

  for (int t0 = t_begin + wave * 64; t0 < t_end; t0 += 256) {
    const int t = t0 + lane;
    const bool valid = t < t_end;
    const int tc = valid ? t : t_end - 1;

    // ---- scores, one lane per token
    float sc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) sc[r] = 0.0f;
    const uint4* kp = reinterpret_cast<const uint4*>(kbase + (int64_t)tc * D);
#pragma unroll 2
    for (int c = 0; c < D / 8; ++c) {
      float kf[8];
      bf16x8_to_f32(kp[c], kf);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[r] = fmaf(qs[r][8 * c + e], kf[e], sc[r]);
      }
    }
    if constexpr (RESID) {
      for (int li = 0; li < a.n_loops_launch; ++li) {
        const int bits = a.bits[li];
        if (bits == 0) continue;
        const int lo = li * G, hi = lo + G;
        const int64_t vec = (int64_t)bh * S + tc;
        const uint32_t* cw = a.kc[li] + vec * (D * bits / 32);
        const uint16_t* sp = a.ks[li] + vec * NG;
        for (int grp = 0; grp < NG; ++grp) {
          const float s = f16_bits_to_f32(sp[grp]) * RsqrtD<D>::v;
          float part[NR];
#pragma unroll
          for (int r = 0; r < NR; ++r) part[r] = 0.0f;
          for (int e = 0; e < 32; ++e) {
            const float lev = level_any(cw, grp * 32 + e, bits);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
              if (r >= lo && r < hi) part[r] = fmaf(qt[r][grp * 32 + e], lev, part[r]);
            }
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (r >= lo && r < hi) sc[r] = fmaf(s, part[r], sc[r]);
          }
        }
      }
    }

    // ---- online softmax (log2 domain)
    float alpha[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float zz = valid ? sc[r] * a.scale_log2 : -INFINITY;
      const float mx = wave_max(zz);
      const float m_new = fmaxf(m[r], mx);
      alpha[r] = exp2f(m[r] - m_new);  // m = -inf on the first tile -> 0
      const float p = valid ? exp2f(zz - m_new) : 0.0f;
      l[r] = fmaf(l[r], alpha[r], p);
      m[r] = m_new;
      pb[wave][r][lane] = p;
    }
    wave_lds_sync();

    // ---- PV, one lane per output coordinate
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        o_ref[r][j] *= alpha[r];
        if constexpr (RESID) o_res[r][j] *= alpha[r];
      }
    }
    const int ntok = min(64, t_end - t0);
    for (int tt = 0; tt < ntok; ++tt) {
      const int tk = t0 + tt;
      float vv[DJ];
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        const uint16_t vb = vbase[(int64_t)tk * D + lane + 64 * j];
        vv[j] = __uint_as_float((uint32_t)vb << 16);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float p = pb[wave][r][tt];
#pragma unroll
        for (int j = 0; j < DJ; ++j) o_ref[r][j] = fmaf(p, vv[j], o_ref[r][j]);
      }
      if constexpr (RESID) {
        for (int li = 0; li < a.n_loops_launch; ++li) {
          const int bits = a.bits[li];
          if (bits == 0) continue;
          const int lo = li * G, hi = lo + G;
          const int64_t vec = (int64_t)bh * S + tk;
          const uint32_t* cw = a.vc[li] + vec * (D * bits / 32);
          const uint16_t* sp = a.vs[li] + vec * NG;
          float val[DJ];
#pragma unroll
          for (int j = 0; j < DJ; ++j) {
            const int d = lane + 64 * j;
            val[j] = f16_bits_to_f32(sp[d >> 5]) * level_any(cw, d, bits);
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (r >= lo && r < hi) {
              const float p = pb[wave][r][tt];
#pragma unroll
              for (int j = 0; j < DJ; ++j) o_res[r][j] = fmaf(p, val[j], o_res[r][j]);
            }
          }
        }
      }
    }
    wave_lds_sync();
  }

  // ---- merge the four waves (fixed order, so results are reproducible)
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float ls = wave_sum(l[r]);
    if (lane == 0) {
      mw[wave][r] = m[r];
      lw[wave][r] = ls;
    }
  }
  __syncthreads();
  float* acc_ref = &pb[0][0][0];       // reuse: NR * D floats
  float* acc_res = acc_ref + NR * D;   // NR * D floats (fits: 2 * NR * D <= 4 * NR * 64)
  float fw[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, mw[w][r]);
    fw[r] = (m[r] == -INFINITY) ? 0.0f : exp2f(m[r] - mm);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
          const int d = lane + 64 * j;
          const float vr = fw[r] * o_ref[r][j];
          float vs = 0.0f;
          if constexpr (RESID) vs = fw[r] * o_res[r][j];
          if (w == 0) {
            acc_ref[r * D + d] = vr;
            acc_res[r * D + d] = vs;
          } else {
            acc_ref[r * D + d] += vr;
            acc_res[r * D + d] += vs;
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
        const int lo = (k / h) * 2 * h + (k % h);
        const float x = acc_res[r * D + lo], y = acc_res[r * D + lo + h];
        acc_res[r * D + lo] = x + y;
        acc_res[r * D + lo + h] = x - y;
      }
      __syncthreads();
    }
  }
  // ---- write partials
  for (int i = threadIdx.x; i < R * (D + 2); i += 256) {
    const int r = i / (D + 2), e = i % (D + 2);
    const int loop = a.loop_base + r / G + z;
    const int hq = kvh * G + r % G;
    float* dst = a.ws + ((((int64_t)loop * a.batch + b) * a.n_q_heads + hq) * a.n_splits + split) * (D + 2);
    float val;
    if (e == 0) {
      float mm = -INFINITY;
      for (int w = 0; w < 4; ++w) mm = fmaxf(mm, mw[w][r]);
      val = mm;
    } else if (e == 1) {
      float mm = -INFINITY;
      for (int w = 0; w < 4; ++w) mm = fmaxf(mm, mw[w][r]);
      float ls = 0.0f;
      for (int w = 0; w < 4; ++w) ls += (mw[w][r] == -INFINITY) ? 0.0f : exp2f(mw[w][r] - mm) * lw[w][r];
      val = ls;
    } else {
      const int d = e - 2;
      val = acc_ref[r * D + d] + (RESID ? acc_res[r * D + d] * RsqrtD<D>::v : 0.0f);
    }
    dst[e] = val;
  }
}

// One wave per output row: merge the splits by log-sum-exp and normalise.
template <int D>
__global__ __launch_bounds__(256) void rq_combine_kernel(CombineArgs a) {
  constexpr int DJ = D / 64;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.n_out) return;
  const float* src = a.ws + row * a.n_splits * (D + 2);
  float mm = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) mm = fmaxf(mm, src[s * (D + 2)]);
  float lsum = 0.0f, o[DJ];
#pragma unroll
  for (int j = 0; j < DJ; ++j) o[j] = 0.0f;
  for (int s = 0; s < a.n_splits; ++s) {
    const float* p = src + s * (D + 2);
    const float w = (p[0] == -INFINITY) ? 0.0f : exp2f(p[0] - mm);
    lsum = fmaf(w, p[1], lsum);
#pragma unroll
    for (int j = 0; j < DJ; ++j) o[j] = fmaf(w, p[2 + lane + 64 * j], o[j]);
  }
  const float inv = 1.0f / lsum;
  float* dst = a.out + row * D;
#pragma unroll
  for (int j = 0; j < DJ; ++j) dst[lane + 64 * j] = o[j] * inv;
}

template <int D, bool RESID>
static void launch_partial_nr(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  if (a.n_rows <= 4) hipLaunchKernelGGL((rq_decode_partial_v1<D, 4, RESID>), grid, dim3(256), 0, stream, a);
  else if (a.n_rows <= 8) hipLaunchKernelGGL((rq_decode_partial_v1<D, 8, RESID>), grid, dim3(256), 0, stream, a);
  else if (a.n_rows <= 16) hipLaunchKernelGGL((rq_decode_partial_v1<D, 16, RESID>), grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((rq_decode_partial_v1<D, 32, RESID>), grid, dim3(256), 0, stream, a);
}

hipError_t launch_decode_partial(const DecodeArgs& a, int head_dim, int n_z, bool residual, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.n_splits * a.batch * a.n_kv_heads), n_z);
  if (head_dim == 128) {
    if (residual) launch_partial_nr<128, true>(a, grid, stream);
    else launch_partial_nr<128, false>(a, grid, stream);
  } else {
    if (residual) launch_partial_nr<64, true>(a, grid, stream);
    else launch_partial_nr<64, false>(a, grid, stream);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n_out + 3) / 4));
  if (head_dim == 128) hipLaunchKernelGGL(rq_combine_kernel<128>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(rq_combine_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rq
