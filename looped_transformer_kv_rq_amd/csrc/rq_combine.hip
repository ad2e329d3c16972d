// Log-sum-exp merge of the split-S decode partials.
//
// A partial holds, for one query row and one token range, the running maximum
// of the scores (log2 units), the sum of exp2(score - max), the unnormalised
// reference output and, for residual loops, the unnormalised residual output
// in the rotated domain. The merge rescales every split to the common maximum
// in a fixed split order, so the result does not depend on scheduling. It
// then applies the normalised Walsh-Hadamard rotation to the merged residual
// accumulator once, because H sum(p (s*lev)) = sum(p H (s*lev)), and divides
// by the total weight.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

// One wave per output row; lane owns coordinates lane + 64 j.
template <int D>
__global__ __launch_bounds__(256) void rq_combine_kernel(CombineArgs a) {
  constexpr int DJ = D / 64;
  constexpr int REC = 2 * D + 2;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.n_out) return;
  const float* src = a.ws + row * a.n_splits * REC;
  // Records to merge: all n_splits, or (length-balanced splits) sequence b's
  // own split count, then the tail record if there is one.
  int n_pre = a.n_splits, n_vis = a.n_splits;
  if (a.row_splits != nullptr) {
    const int bb = (int)((row / a.n_q_heads) % a.batch);
    n_pre = min(a.row_splits[bb], a.n_splits);
    n_vis = n_pre + (a.tail_slot >= 0 ? 1 : 0);
  }
  // Splits go in chunks of kChunk whose loads are all issued before any is
  // used; the running maximum and the sums are rescaled chunk by chunk, in
  // split order, so the result does not depend on scheduling.
  constexpr int kChunk = 8;
  float mm = -INFINITY, lsum = 0.0f, o[DJ], r[DJ];
#pragma unroll
  for (int j = 0; j < DJ; ++j) o[j] = r[j] = 0.0f;
  for (int s0 = 0; s0 < n_vis; s0 += kChunk) {
    float pm[kChunk], pl[kChunk], po[kChunk][DJ], pr[kChunk][DJ];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const bool in = s0 + c < n_vis;
      const int v = in ? s0 + c : s0;
      const float* p = src + (v < n_pre ? v : a.tail_slot) * REC;
      pm[c] = in ? p[0] : -INFINITY;
      pl[c] = p[1];
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        po[c][j] = p[2 + lane + 64 * j];
        pr[c][j] = a.residual ? p[2 + D + lane + 64 * j] : 0.0f;
      }
    }
    float cm = mm;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) cm = fmaxf(cm, pm[c]);
    if (cm == -INFINITY) continue;  // no position yet
    const float keep = mm == -INFINITY ? 0.0f : exp2f(mm - cm);
    lsum *= keep;
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
      o[j] *= keep;
      r[j] *= keep;
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const float w = pm[c] == -INFINITY ? 0.0f : exp2f(pm[c] - cm);
      lsum = fmaf(w, pl[c], lsum);
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        o[j] = fmaf(w, po[c][j], o[j]);
        r[j] = fmaf(w, pr[c][j], r[j]);
      }
    }
    mm = cm;
  }
  if (a.residual) {
    // unnormalised transform: index bit 6 in the lane, bits 0..5 across lanes
    if constexpr (DJ == 2) {
      const float x = r[0], y = r[1];
      r[0] = x + y;
      r[1] = x - y;
    }
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const bool upper = (lane & s) != 0;
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        const float p = __shfl_xor(r[j], s);
        r[j] = upper ? p - r[j] : r[j] + p;
      }
    }
#pragma unroll
    for (int j = 0; j < DJ; ++j) o[j] = fmaf(r[j], RsqrtD<D>::v, o[j]);
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;  // no position at all: a zero row
  float* dst = a.out + row * D;
#pragma unroll
  for (int j = 0; j < DJ; ++j) dst[lane + 64 * j] = o[j] * inv;
}

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n_out + 3) / 4));
  if (head_dim == 128) hipLaunchKernelGGL(rq_combine_kernel<128>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(rq_combine_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rq
