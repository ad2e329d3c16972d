// C ABI of librq: argument checks (host only, before any HIP call), split
// planning, and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "rq.h"
#include "rq_internal.h"

namespace {

using namespace rq;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// residual code widths of the format: 2 and 4, and 3 and 8 for per-(layer, loop) tables
bool residual_width(int32_t b) { return b == 2 || b == 3 || b == 4 || b == 8; }

// RQ_OK, RQ_EINVAL or RQ_EUNSUPPORTED
int check_shape(const rq_shape* s) {
  if (s == nullptr) return RQ_EINVAL;
  if (s->batch <= 0 || s->n_kv_heads <= 0 || s->seq_len <= 0 || s->head_dim <= 0) return RQ_EINVAL;
  if (s->head_dim != 64 && s->head_dim != 128) return RQ_EUNSUPPORTED;
  return RQ_OK;
}

int64_t n_vectors(const rq_shape* s) { return (int64_t)s->batch * s->n_kv_heads * s->seq_len; }

int check_heads(const rq_shape* s, int32_t n_q_heads, int32_t n_loops) {
  int st = check_shape(s);
  if (st != RQ_OK) return st;
  if (n_q_heads <= 0 || n_q_heads % s->n_kv_heads != 0) return RQ_EINVAL;
  if (n_loops < 1 || n_loops > kMaxLoops) return RQ_EINVAL;
  if (n_q_heads / s->n_kv_heads > 32) return RQ_EUNSUPPORTED;
  // the decode addresses one (batch, kv head) row of the cache with 32-bit byte offsets
  if ((int64_t)s->seq_len * 2 * s->head_dim > INT32_MAX) return RQ_EUNSUPPORTED;
  return RQ_OK;
}

// Automatic split count. The partial blocks of a launch run in rounds of as
// many as the device holds at once: two 4-wave blocks per CU (one 16-row set),
// four 2-wave blocks (paired sets, more than 16 query rows of at most 16 per
// kv head) or one (32-row blocks, more than 16 query heads per kv head), on
// 256 CUs. A 16-row launch whose four waves stage more than half a CU's LDS
// per tile (INT8 loops, or several INT4 loops) also holds one block per CU. A
// round that is only partly full leaves CUs idle for a whole block time, and
// every block also pays a fixed start and merge (taken as 6 tiles of tokens).
// The plan takes the split count with the least modelled time,
//   ceil(rows * n / round) * (1 / n + 6 * 64 / seq_len)   (in row times),
// the smallest such n on ties. This keeps the best points of split sweeps on
// l4_b16_s4k (4) and mixed_s32k (8; 4 with an INT8 loop), and at the peak
// batch (10,720 rows in rounds of 1,024 blocks) takes 2 splits, whose 21
// rounds of half-length blocks end 5% sooner than 11 full-length ones. A
// split never holds fewer tokens than one 64-token unit.

struct SplitPlan {
  int32_t n_splits;
  int32_t tokens_per_split;
};

// Blocks per round for a call with these loop widths (bits: host [n_loops],
// or nullptr for widths whose 16-row blocks fit two to a CU). Of a 16-row
// call the first launch decides: it holds as many loops as four waves' tiles
// fit in one block's LDS.
int64_t round_blocks(const rq_shape* s, int32_t n_q_heads, int32_t n_loops, const int32_t* bits) {
  const int64_t G = n_q_heads / s->n_kv_heads;
  if (G > 16) return 256;
  if (G * n_loops > 16) return 1024;
  if (bits != nullptr) {
    int32_t first[kMaxLoops];
    int nl = 0;
    for (int i = 0; i < n_loops && i < kMaxLoops; ++i) {
      first[nl] = bits[i];
      if (nl > 0 && 4 * decode_wave_lds_bytes(s->head_dim, first, nl + 1) > kMaxBlockLds) break;
      ++nl;
    }
    if (8 * decode_wave_lds_bytes(s->head_dim, first, nl) > kMaxBlockLds) return 256;
  }
  return 512;
}

// The split count a request of n gives: splits of a whole number of 64-token
// units, as few as hold the positions.
static SplitPlan realize_splits(int64_t seq_len, int64_t n) {
  const int64_t max_splits = (seq_len + kDecodeTile - 1) / kDecodeTile;
  if (n < 1) n = 1;
  if (n > max_splits) n = max_splits;
  int64_t tps = (seq_len + n - 1) / n;
  tps = (tps + kDecodeTile - 1) / kDecodeTile * kDecodeTile;
  return {(int32_t)((seq_len + tps - 1) / tps), (int32_t)tps};
}

static SplitPlan plan_for_round(const rq_shape* s, int64_t round) {
  const int64_t rows = (int64_t)s->batch * s->n_kv_heads;
  const double fixed = 6.0 * kDecodeTile / (double)s->seq_len;
  SplitPlan best_plan = realize_splits(s->seq_len, 1);
  double best = 0.0;
  for (int64_t c = 1; c <= 64; ++c) {
    const SplitPlan p = realize_splits(s->seq_len, c);
    const int64_t n = p.n_splits;
    const double t = (double)((rows * n + round - 1) / round) * (1.0 / (double)n + fixed);
    if (c == 1 || t < best * (1.0 - 1e-9)) {
      best = t;
      best_plan = p;
    }
  }
  return best_plan;
}

SplitPlan plan_splits(const rq_shape* s, int32_t n_q_heads, int32_t n_loops, const int32_t* bits, int32_t requested) {
  if (requested > 0) return realize_splits(s->seq_len, requested);
  return plan_for_round(s, round_blocks(s, n_q_heads, n_loops, bits));
}

// The most splits an automatic plan takes for any loop widths: what the
// workspace query sizes for
static int32_t max_auto_splits(const rq_shape* s, int32_t n_q_heads, int32_t n_loops, int32_t requested) {
  const SplitPlan p = plan_splits(s, n_q_heads, n_loops, nullptr, requested);
  if (requested > 0 || round_blocks(s, n_q_heads, n_loops, nullptr) != 512) return p.n_splits;
  return std::max(p.n_splits, plan_for_round(s, 256).n_splits);
}

// Workspace: split partials [n_loops][B][Hq][n_splits][2D + 2] floats, padded
// to 256 bytes, then one rotated-query record per query row (written only by
// the calls that run the prep kernel).
size_t partial_bytes(const rq_shape* s, int32_t n_q_heads, int32_t n_loops, int32_t n_splits) {
  const size_t b = (size_t)n_loops * s->batch * n_q_heads * n_splits * (2 * s->head_dim + 2) * sizeof(float);
  return (b + 255) / 256 * 256;
}

size_t workspace_bytes_for(const rq_shape* s, int32_t n_q_heads, int32_t n_loops, int32_t n_splits) {
  return partial_bytes(s, n_q_heads, n_loops, n_splits) +
         (size_t)n_loops * s->batch * n_q_heads * query_prep_bytes(s->head_dim);
}

// A ragged decode with an automatic split count balances its splits over the
// actual prefix lengths (see DecodeArgs::balance_target): up to
// balanced_max_row_splits records per row, plus the split count of every
// sequence (int32 [B]) after the query records.
int32_t balanced_rec_splits(const rq_shape* s, int32_t tail_len) {
  return balanced_max_row_splits((int64_t)s->batch * s->n_kv_heads, s->seq_len) + (tail_len > 0 ? 1 : 0);
}
size_t balanced_workspace_bytes(const rq_shape* s, int32_t n_q_heads, int32_t n_loops, int32_t tail_len) {
  return workspace_bytes_for(s, n_q_heads, n_loops, balanced_rec_splits(s, tail_len)) + 4 * (size_t)s->batch;
}

int hip_status(hipError_t e) { return e == hipSuccess ? RQ_OK : RQ_EHIP; }

int run_combine(const rq_shape* s, int32_t n_q_heads, int32_t n_loops, int32_t n_splits, const float* ws,
                float* out, bool residual, hipStream_t stream, const int32_t* row_splits = nullptr,
                int32_t tail_slot = -1) {
  CombineArgs c{};
  c.ws = ws;
  c.out = out;
  c.n_out = (int64_t)n_loops * s->batch * n_q_heads;
  c.n_splits = n_splits;
  c.residual = residual ? 1 : 0;
  c.row_splits = row_splits;
  c.batch = s->batch;
  c.n_q_heads = n_q_heads;
  c.tail_slot = tail_slot;
  return hip_status(launch_combine(c, s->head_dim, stream));
}

void fill_common(DecodeArgs& a, const rq_shape* s, int32_t n_q_heads, const uint16_t* q, float softmax_scale,
                 const SplitPlan& p, void* workspace) {
  a.q = q;
  a.ws = static_cast<float*>(workspace);
  a.group = n_q_heads / s->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = s->n_kv_heads;
  a.batch = s->batch;
  a.seq_len = s->seq_len;
  a.n_splits = p.n_splits;
  a.tokens_per_split = p.tokens_per_split;
  a.rec_splits = p.n_splits;
  a.split_base = 0;
  a.seq_lens = nullptr;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
}

// Argument checks of an encode (no HIP call).
int encode_check(const rq_shape* shape, int32_t n_loops, const uint16_t* const* x, const int32_t* bits,
                 const uint16_t* ref, uint32_t* const* codes, uint16_t* const* scales, int32_t refits) {
  int st = check_shape(shape);
  if (st != RQ_OK) return st;
  if (n_loops < 1 || n_loops > kMaxLoops) return RQ_EINVAL;
  if (refits < 0 || refits > RQ_MAX_REFITS) return RQ_EINVAL;
  if (x == nullptr || bits == nullptr || codes == nullptr || scales == nullptr) return RQ_EINVAL;
  for (int i = 0; i < n_loops; ++i) {
    if (x[i] == nullptr || codes[i] == nullptr || scales[i] == nullptr) return RQ_EINVAL;
  }
  for (int i = 0; i < n_loops; ++i) {
    if (!residual_width(bits[i])) return RQ_EUNSUPPORTED;
  }
  if (ref != nullptr && !aligned16(ref)) return RQ_EALIGN;
  for (int i = 0; i < n_loops; ++i) {
    if (!aligned16(x[i]) || !aligned16(codes[i]) || !aligned16(scales[i])) return RQ_EALIGN;
  }
  return RQ_OK;
}

// Checks one tensor's encode and fills its launch arguments (no HIP call).
// ref = the final loop, or NULL for the rotation-only baseline (a zero
// reference, so each state is quantized directly after the rotation).
int encode_fill(const rq_shape* shape, int32_t n_loops, const uint16_t* const* x, const int32_t* bits,
                const uint16_t* ref, uint32_t* const* codes, uint16_t* const* scales, int32_t refits,
                EncodeArgs& a) {
  const int st = encode_check(shape, n_loops, x, bits, ref, codes, scales, refits);
  if (st != RQ_OK) return st;
  a = EncodeArgs{};
  for (int i = 0; i < n_loops; ++i) {
    a.x[i] = x[i];
    a.codes[i] = codes[i];
    a.scales[i] = scales[i];
    a.bits[i] = bits[i];
  }
  a.ref = ref;
  a.n_loops = n_loops;
  a.refits = refits;
  a.n_vec = n_vectors(shape);
  return RQ_OK;
}

int encode_common(const rq_shape* shape, int32_t n_loops, const uint16_t* const* x, const int32_t* bits,
                  const uint16_t* ref, uint32_t* const* codes, uint16_t* const* scales, int32_t refits,
                  void* stream) {
  EncodeArgs a;
  const int st = encode_fill(shape, n_loops, x, bits, ref, codes, scales, refits, a);
  if (st != RQ_OK) return st;
  return hip_status(launch_encode(&a, 1, shape->head_dim, static_cast<hipStream_t>(stream)));
}

int reconstruct_common(const rq_shape* shape, int32_t bits, const uint16_t* ref, const uint32_t* codes,
                       const uint16_t* scales, int32_t out_dtype, void* out, void* stream) {
  int st = check_shape(shape);
  if (st != RQ_OK) return st;
  if (out == nullptr) return RQ_EINVAL;
  if (bits != 0 && !residual_width(bits)) return RQ_EUNSUPPORTED;
  if (out_dtype != RQ_OUT_F32 && out_dtype != RQ_OUT_BF16) return RQ_EUNSUPPORTED;
  if (bits != 0 && (codes == nullptr || scales == nullptr)) return RQ_EINVAL;
  if ((ref != nullptr && !aligned16(ref)) || !aligned16(out)) return RQ_EALIGN;
  if (bits != 0 && (!aligned16(codes) || !aligned16(scales))) return RQ_EALIGN;
  ReconstructArgs a{};
  a.ref = ref;
  a.codes = codes;
  a.scales = scales;
  a.out = out;
  a.n_vec = n_vectors(shape);
  return hip_status(launch_reconstruct(a, shape->head_dim, bits, out_dtype == RQ_OUT_BF16,
                                       static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int rq_encode(const rq_shape* shape, int32_t n_loops, const uint16_t* const* x, const int32_t* bits,
              const uint16_t* ref, uint32_t* const* codes, uint16_t* const* scales, void* stream) {
  if (ref == nullptr) return RQ_EINVAL;
  return encode_common(shape, n_loops, x, bits, ref, codes, scales, 0, stream);
}

int rq_encode_kv(const rq_shape* shape, int32_t n_loops, const uint16_t* const* kx, const uint16_t* const* vx,
                 const int32_t* bits, const uint16_t* k_ref, const uint16_t* v_ref, uint32_t* const* k_codes,
                 uint16_t* const* k_scales, uint32_t* const* v_codes, uint16_t* const* v_scales, void* stream) {
  if (k_ref == nullptr || v_ref == nullptr) return RQ_EINVAL;
  EncodeArgs a[2];
  int st = encode_fill(shape, n_loops, kx, bits, k_ref, k_codes, k_scales, 0, a[0]);
  if (st != RQ_OK) return st;
  st = encode_fill(shape, n_loops, vx, bits, v_ref, v_codes, v_scales, 0, a[1]);
  if (st != RQ_OK) return st;
  return hip_status(launch_encode(a, 2, shape->head_dim, static_cast<hipStream_t>(stream)));
}

int rq_encode_refit(const rq_shape* shape, int32_t n_loops, const uint16_t* const* x, const int32_t* bits,
                    const uint16_t* ref, uint32_t* const* codes, uint16_t* const* scales, int32_t refits,
                    void* stream) {
  if (ref == nullptr) return RQ_EINVAL;
  return encode_common(shape, n_loops, x, bits, ref, codes, scales, refits, stream);
}

int rq_reconstruct(const rq_shape* shape, int32_t bits, const uint16_t* ref, const uint32_t* codes,
                   const uint16_t* scales, int32_t out_dtype, void* out, void* stream) {
  if (ref == nullptr) return RQ_EINVAL;
  return reconstruct_common(shape, bits, ref, codes, scales, out_dtype, out, stream);
}

}  // extern "C"

namespace {

// RQ_OK if `pages` describes a paged cache of capacity shape->seq_len.
int check_pages(const rq_shape* shape, const rq_pages* pages) {
  if (pages == nullptr || pages->block_table == nullptr) return RQ_EINVAL;
  const int32_t p = pages->block_size;
  if (p < 64 || (p & (p - 1)) != 0) return RQ_EUNSUPPORTED;
  if (pages->max_blocks < 1 || pages->n_blocks < 1) return RQ_EINVAL;
  if ((int64_t)pages->max_blocks * p != shape->seq_len) return RQ_EINVAL;
  if (!aligned16(pages->block_table)) return RQ_EALIGN;
  return RQ_OK;
}

int log2_of(int32_t p) {
  int l = 0;
  while ((1 << l) < p) ++l;
  return l;
}

// Checks one tensor's append and fills its launch arguments (no HIP call).
int append_fill(const rq_shape* cache, const rq_pages* pages, int32_t n_loops, int32_t t_new,
                const uint16_t* const* x, const int32_t* bits, const uint16_t* ref_new, const int32_t* pos,
                uint16_t* ref_cache, uint32_t* const* codes, uint16_t* const* scales, EncodeArgs& a) {
  int st = check_shape(cache);
  if (st != RQ_OK) return st;
  if (pages != nullptr) {
    st = check_pages(cache, pages);
    if (st != RQ_OK) return st;
  }
  if (n_loops < 1 || n_loops > kMaxLoops || t_new < 1) return RQ_EINVAL;
  if (x == nullptr || bits == nullptr || ref_new == nullptr || pos == nullptr || ref_cache == nullptr ||
      codes == nullptr || scales == nullptr)
    return RQ_EINVAL;
  for (int i = 0; i < n_loops; ++i) {
    if (x[i] == nullptr || codes[i] == nullptr || scales[i] == nullptr) return RQ_EINVAL;
  }
  for (int i = 0; i < n_loops; ++i) {
    if (!residual_width(bits[i])) return RQ_EUNSUPPORTED;
  }
  if (!aligned16(ref_new) || !aligned16(ref_cache)) return RQ_EALIGN;
  for (int i = 0; i < n_loops; ++i) {
    if (!aligned16(x[i]) || !aligned16(codes[i]) || !aligned16(scales[i])) return RQ_EALIGN;
  }
  a = EncodeArgs{};
  for (int i = 0; i < n_loops; ++i) {
    a.x[i] = x[i];
    a.codes[i] = codes[i];
    a.scales[i] = scales[i];
    a.bits[i] = bits[i];
  }
  a.ref = ref_new;
  a.n_loops = n_loops;
  a.pos = pos;
  a.t_new = t_new;
  a.n_kv_heads = cache->n_kv_heads;
  a.s_cap = cache->seq_len;
  a.ref_out = ref_cache;
  if (pages != nullptr) {
    a.block_table = pages->block_table;
    a.max_blocks = pages->max_blocks;
    a.log2_block = log2_of(pages->block_size);
    a.n_blocks = pages->n_blocks;
  }
  a.n_vec = (int64_t)cache->batch * cache->n_kv_heads * t_new;
  return RQ_OK;
}

int append_impl(const rq_shape* cache, const rq_pages* pages, int32_t n_loops, int32_t t_new,
                const uint16_t* const* x, const int32_t* bits, const uint16_t* ref_new, const int32_t* pos,
                uint16_t* ref_cache, uint32_t* const* codes, uint16_t* const* scales, void* stream) {
  EncodeArgs a;
  const int st = append_fill(cache, pages, n_loops, t_new, x, bits, ref_new, pos, ref_cache, codes, scales, a);
  if (st != RQ_OK) return st;
  return hip_status(launch_encode(&a, 1, cache->head_dim, static_cast<hipStream_t>(stream)));
}

// K and V of one append in one launch
int append_kv_impl(const rq_shape* cache, const rq_pages* pages, int32_t n_loops, int32_t t_new,
                   const uint16_t* const* kx, const uint16_t* const* vx, const int32_t* bits,
                   const uint16_t* k_ref_new, const uint16_t* v_ref_new, const int32_t* pos, uint16_t* k_ref_cache,
                   uint16_t* v_ref_cache, uint32_t* const* k_codes, uint16_t* const* k_scales,
                   uint32_t* const* v_codes, uint16_t* const* v_scales, void* stream) {
  EncodeArgs a[2];
  int st = append_fill(cache, pages, n_loops, t_new, kx, bits, k_ref_new, pos, k_ref_cache, k_codes, k_scales, a[0]);
  if (st != RQ_OK) return st;
  st = append_fill(cache, pages, n_loops, t_new, vx, bits, v_ref_new, pos, v_ref_cache, v_codes, v_scales, a[1]);
  if (st != RQ_OK) return st;
  return hip_status(launch_encode(a, 2, cache->head_dim, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int rq_encode_append(const rq_shape* cache, int32_t n_loops, int32_t t_new, const uint16_t* const* x,
                     const int32_t* bits, const uint16_t* ref_new, const int32_t* pos, uint16_t* ref_cache,
                     uint32_t* const* codes, uint16_t* const* scales, void* stream) {
  return append_impl(cache, nullptr, n_loops, t_new, x, bits, ref_new, pos, ref_cache, codes, scales, stream);
}

int rq_encode_append_paged(const rq_shape* cache, const rq_pages* pages, int32_t n_loops, int32_t t_new,
                           const uint16_t* const* x, const int32_t* bits, const uint16_t* ref_new,
                           const int32_t* pos, uint16_t* ref_pages, uint32_t* const* codes,
                           uint16_t* const* scales, void* stream) {
  if (pages == nullptr) return RQ_EINVAL;
  return append_impl(cache, pages, n_loops, t_new, x, bits, ref_new, pos, ref_pages, codes, scales, stream);
}

int rq_encode_append_kv(const rq_shape* cache, int32_t n_loops, int32_t t_new, const uint16_t* const* kx,
                        const uint16_t* const* vx, const int32_t* bits, const uint16_t* k_ref_new,
                        const uint16_t* v_ref_new, const int32_t* pos, uint16_t* k_ref_cache, uint16_t* v_ref_cache,
                        uint32_t* const* k_codes, uint16_t* const* k_scales, uint32_t* const* v_codes,
                        uint16_t* const* v_scales, void* stream) {
  return append_kv_impl(cache, nullptr, n_loops, t_new, kx, vx, bits, k_ref_new, v_ref_new, pos, k_ref_cache,
                        v_ref_cache, k_codes, k_scales, v_codes, v_scales, stream);
}

int rq_encode_append_paged_kv(const rq_shape* cache, const rq_pages* pages, int32_t n_loops, int32_t t_new,
                              const uint16_t* const* kx, const uint16_t* const* vx, const int32_t* bits,
                              const uint16_t* k_ref_new, const uint16_t* v_ref_new, const int32_t* pos,
                              uint16_t* k_ref_pages, uint16_t* v_ref_pages, uint32_t* const* k_codes,
                              uint16_t* const* k_scales, uint32_t* const* v_codes, uint16_t* const* v_scales,
                              void* stream) {
  if (pages == nullptr) return RQ_EINVAL;
  return append_kv_impl(cache, pages, n_loops, t_new, kx, vx, bits, k_ref_new, v_ref_new, pos, k_ref_pages,
                        v_ref_pages, k_codes, k_scales, v_codes, v_scales, stream);
}

int rq_encode_layers(const rq_shape* shape, int32_t n_layers, int32_t n_loops, const uint16_t* const* x,
                     const int32_t* bits_table, const uint16_t* const* ref, uint32_t* const* codes,
                     uint16_t* const* scales, void* stream) {
  if (n_layers < 1 || n_layers > RQ_MAX_LAYERS || n_loops < 1 || n_loops > kMaxLoops) return RQ_EINVAL;
  if (x == nullptr || bits_table == nullptr || ref == nullptr || codes == nullptr || scales == nullptr)
    return RQ_EINVAL;
  for (int l = 0; l < n_layers; ++l) {
    if (ref[l] == nullptr) return RQ_EINVAL;
    const int64_t o = (int64_t)l * n_loops;
    const int st = encode_check(shape, n_loops, x + o, bits_table + o, ref[l], codes + o, scales + o, 0);
    if (st != RQ_OK) return st;
  }
  // layers go two to a launch
  for (int l = 0; l < n_layers; l += 2) {
    const int n = n_layers - l < 2 ? n_layers - l : 2;
    EncodeArgs a[2];
    for (int j = 0; j < n; ++j) {
      const int64_t o = (int64_t)(l + j) * n_loops;
      const int st = encode_fill(shape, n_loops, x + o, bits_table + o, ref[l + j], codes + o, scales + o, 0, a[j]);
      if (st != RQ_OK) return st;
    }
    const int st = hip_status(launch_encode(a, n, shape->head_dim, static_cast<hipStream_t>(stream)));
    if (st != RQ_OK) return st;
  }
  return RQ_OK;
}

int rq_encode_rotonly(const rq_shape* shape, int32_t n_states, const uint16_t* const* x, const int32_t* bits,
                      uint32_t* const* codes, uint16_t* const* scales, void* stream) {
  return encode_common(shape, n_states, x, bits, nullptr, codes, scales, 0, stream);
}

int rq_reconstruct_rotonly(const rq_shape* shape, int32_t bits, const uint32_t* codes, const uint16_t* scales,
                           int32_t out_dtype, void* out, void* stream) {
  if (bits == 0) return RQ_EUNSUPPORTED;
  return reconstruct_common(shape, bits, nullptr, codes, scales, out_dtype, out, stream);
}

int32_t rq_decode_attn_splits(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const int32_t* bits,
                              int32_t n_splits) {
  if (check_heads(shape, n_q_heads, n_loops) != RQ_OK || n_splits < 0) return 0;
  if (bits != nullptr) {
    for (int i = 0; i < n_loops; ++i) {
      if (bits[i] != 0 && !residual_width(bits[i])) return 0;
    }
  }
  return plan_splits(shape, n_q_heads, n_loops, bits, n_splits).n_splits;
}

size_t rq_decode_attn_workspace(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, int32_t n_splits) {
  if (check_heads(shape, n_q_heads, n_loops) != RQ_OK || n_splits < 0) return 0;
  return workspace_bytes_for(shape, n_q_heads, n_loops, max_auto_splits(shape, n_q_heads, n_loops, n_splits));
}

}  // extern "C"

namespace {

// The residual-cache decode. seq_lens (device [B], or NULL for all seq_len)
// bounds each sequence's prefix; tail_len > 0 adds tail_len bf16 positions per
// loop (tail_k / tail_v), merged as one more split.
int decode_impl(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                const uint16_t* k_ref, const uint16_t* v_ref, const rq_loop_view* loops, const int32_t* seq_lens,
                int32_t tail_len, const uint16_t* const* tail_k, const uint16_t* const* tail_v,
                float softmax_scale, int32_t n_splits, float* out, void* workspace, size_t workspace_bytes,
                void* stream, const rq_pages* pages = nullptr) {
  int st = check_heads(shape, n_q_heads, n_loops);
  if (st != RQ_OK) return st;
  if (pages != nullptr) {
    st = check_pages(shape, pages);
    if (st != RQ_OK) return st;
  }
  if (q == nullptr || k_ref == nullptr || v_ref == nullptr || loops == nullptr || out == nullptr) return RQ_EINVAL;
  if (n_splits < 0 || !isfinite(softmax_scale) || tail_len < 0) return RQ_EINVAL;
  if (tail_len > 0) {
    if (tail_k == nullptr || tail_v == nullptr) return RQ_EINVAL;
    for (int i = 0; i < n_loops; ++i) {
      if (tail_k[i] == nullptr || tail_v[i] == nullptr) return RQ_EINVAL;
    }
    rq_shape ts = *shape;
    ts.seq_len = tail_len;
    if (check_heads(&ts, n_q_heads, n_loops) != RQ_OK) return RQ_EUNSUPPORTED;
  }
  for (int i = 0; i < n_loops; ++i) {
    const rq_loop_view& lv = loops[i];
    if (lv.bits != 0 && !residual_width(lv.bits)) return RQ_EUNSUPPORTED;
    if (lv.bits != 0 && (lv.k_codes == nullptr || lv.k_scales == nullptr || lv.v_codes == nullptr ||
                         lv.v_scales == nullptr))
      return RQ_EINVAL;
  }
  if (!aligned16(q) || !aligned16(k_ref) || !aligned16(v_ref) || !aligned16(out)) return RQ_EALIGN;
  for (int i = 0; i < n_loops; ++i) {
    const rq_loop_view& lv = loops[i];
    if (lv.bits != 0 && (!aligned16(lv.k_codes) || !aligned16(lv.k_scales) || !aligned16(lv.v_codes) ||
                         !aligned16(lv.v_scales)))
      return RQ_EALIGN;
  }
  if (tail_len > 0) {
    for (int i = 0; i < n_loops; ++i) {
      if (!aligned16(tail_k[i]) || !aligned16(tail_v[i])) return RQ_EALIGN;
    }
  }
  // Ragged prefixes with an automatic split count: length-balanced splits.
  const bool balanced = seq_lens != nullptr && n_splits == 0;
  int32_t widths[kMaxLoops];
  for (int i = 0; i < n_loops; ++i) widths[i] = loops[i].bits;
  const SplitPlan plan = plan_splits(shape, n_q_heads, n_loops, widths, n_splits);
  const int32_t prefix_recs =
      balanced ? balanced_max_row_splits((int64_t)shape->batch * shape->n_kv_heads, shape->seq_len) : plan.n_splits;
  const int32_t rec_splits = prefix_recs + (tail_len > 0 ? 1 : 0);
  const size_t need = balanced ? balanced_workspace_bytes(shape, n_q_heads, n_loops, tail_len)
                               : workspace_bytes_for(shape, n_q_heads, n_loops, rec_splits);
  if (workspace == nullptr || workspace_bytes < need) return RQ_EWORKSPACE;
  if (!aligned16(workspace)) return RQ_EALIGN;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = n_q_heads / shape->n_kv_heads;
  unsigned char* prep = static_cast<unsigned char*>(workspace) + partial_bytes(shape, n_q_heads, n_loops, rec_splits);
  // balanced: the split count of every sequence, after the query records
  int32_t* row_splits =
      balanced ? reinterpret_cast<int32_t*>(static_cast<unsigned char*>(workspace) +
                                            workspace_bytes_for(shape, n_q_heads, n_loops, rec_splits))
               : nullptr;
  bool any_residual = false;
  for (int i = 0; i < n_loops; ++i) any_residual = any_residual || loops[i].bits != 0;
  struct Launch {
    DecodeArgs sets[kMaxSets];
    int n_sets;
    bool residual;
  };
  Launch launches[kMaxLoops];
  int n_launches = 0;
  // A launch holds at most 32 query rows per kv head, and what its waves stage
  // per tile must fit the block's LDS. Past 16 rows (G <= 16) it runs as two
  // argument sets of at most 16 / G loops each. Further loops go to further
  // launches (each streams the reference again).
  int base = 0;
  while (base < n_loops) {
    int nl = 0;
    int32_t bits[kMaxLoops];
    while (base + nl < n_loops && (nl + 1) * G <= 32) {
      bits[nl] = loops[base + nl].bits;
      if (nl > 0 && 4 * decode_wave_lds_bytes(shape->head_dim, bits, nl + 1) > kMaxBlockLds) break;
      if ((nl + 1) * G > 16 && G <= 16 && nl + 1 > 2 * (16 / G)) break;
      ++nl;
    }
    if (nl == 0) nl = 1;  // G == 32: one loop per launch
    // More than 16 rows whose loops each fit 16: two argument sets of at most
    // 16 / G loops (one 16-row MFMA block each), the loops dealt to balance
    // the LDS each set stages per tile. Otherwise one set.
    int members[kMaxSets][kMaxLoops];
    int n_members[kMaxSets] = {0, 0};
    int n_sets = 1;
    if (nl * G > 16 && G <= 16) {
      n_sets = 2;
      const int cap = 16 / G;
      int order[kMaxLoops];
      for (int j = 0; j < nl; ++j) order[j] = base + j;
      std::stable_sort(order, order + nl, [&](int x, int y) {
        return decode_loop_lds_bytes(shape->head_dim, loops[x].bits) > decode_loop_lds_bytes(shape->head_dim, loops[y].bits);
      });
      int bytes[kMaxSets] = {0, 0};
      for (int j = 0; j < nl; ++j) {
        const int t = (n_members[0] < cap && (n_members[1] >= cap || bytes[0] <= bytes[1])) ? 0 : 1;
        members[t][n_members[t]++] = order[j];
        bytes[t] += decode_loop_lds_bytes(shape->head_dim, loops[order[j]].bits);
      }
    } else {
      for (int j = 0; j < nl; ++j) members[0][j] = base + j;
      n_members[0] = nl;
    }
    DecodeArgs sets[kMaxSets];
    bool residual = false;
    for (int si = 0; si < n_sets; ++si) {
      DecodeArgs& a = sets[si];
      a = DecodeArgs{};
      fill_common(a, shape, n_q_heads, q, softmax_scale, plan, workspace);
      a.rec_splits = rec_splits;
      a.seq_lens = seq_lens;
      if (balanced) {
        a.balance_target = (int32_t)balanced_max_blocks((int64_t)shape->batch * shape->n_kv_heads,
                                                        shape->n_kv_heads, shape->seq_len);
        a.max_row_splits = prefix_recs;
        a.row_splits = row_splits;
      }
      a.qprep = prep;
      a.k[0] = k_ref;
      a.v[0] = v_ref;
      if (pages != nullptr) {
        a.block_table = pages->block_table;
        a.max_blocks = pages->max_blocks;
        a.log2_block = log2_of(pages->block_size);
        a.n_blocks = pages->n_blocks;
      }
      a.n_loops_launch = n_members[si];
      a.n_rows = n_members[si] * G;
      // slots in the order INT8, INT4, INT3, INT2, reference-only: the kernel
      // runs one branch-free loop per width
      int li = 0;
      for (const int want : {8, 4, 3, 2, 0}) {
        for (int j = 0; j < n_members[si]; ++j) {
          const int l = members[si][j];
          const rq_loop_view& lv = loops[l];
          if (lv.bits != want) continue;
          a.loop_id[li] = l;
          a.bits[li] = lv.bits;
          a.slot[li] = SlotPtrs{lv.k_codes, lv.k_scales, lv.v_codes, lv.v_scales};
          if (want == 8) ++a.n8;
          if (want == 4) ++a.n4;
          if (want == 3) ++a.n3;
          if (want == 2) ++a.n2;
          residual = residual || lv.bits != 0;
          ++li;
        }
      }
    }
    for (int si = 0; si < n_sets; ++si) sets[si].zero_residual = any_residual && !residual;
    Launch& ln = launches[n_launches++];
    for (int si = 0; si < n_sets; ++si) ln.sets[si] = sets[si];
    ln.n_sets = n_sets;
    ln.residual = residual;
    base += nl;
  }
  // The residual launches rotate the queries themselves when every one of
  // them can (one 16-row block per set of four waves, a dense cache, INT2 /
  // INT4 loops) and the rotated operands fit their blocks' LDS without costing
  // a block per CU; otherwise one prep kernel writes every query row's record
  // first.
  bool rotate = pages == nullptr;
  for (int i = 0; i < n_launches; ++i) {
    const Launch& ln = launches[i];
    if (!ln.residual) continue;
    int rows = 0;
    for (int si = 0; si < ln.n_sets; ++si) {
      rows = std::max(rows, ln.sets[si].n_rows);
      if (ln.sets[si].n8 + ln.sets[si].n3 > 0) rotate = false;
    }
    const int with = decode_launch_lds_bytes(ln.sets, ln.n_sets, shape->head_dim, true, true);
    const int without = decode_launch_lds_bytes(ln.sets, ln.n_sets, shape->head_dim, true, false);
    if (ln.n_sets == 2 || rows > 16 || with > kMaxBlockLds || kMaxBlockLds / with < kMaxBlockLds / without ||
        decode_launch_waves(ln.sets, ln.n_sets, shape->head_dim, true) != 4)
      rotate = false;
  }
  if (any_residual && !rotate) {
    QueryPrepArgs qa{};
    qa.q = q;
    qa.out = prep;
    for (int i = 0; i < n_loops; ++i) qa.bits[i] = loops[i].bits;
    qa.n_rows = (int64_t)n_loops * shape->batch * n_q_heads;
    qa.batch = shape->batch;
    qa.n_q_heads = n_q_heads;
    st = hip_status(launch_query_prep(qa, shape->head_dim, s));
    if (st != RQ_OK) return st;
  }
  for (int i = 0; i < n_launches; ++i) {
    Launch& ln = launches[i];
    for (int si = 0; si < ln.n_sets; ++si) ln.sets[si].qprep = rotate ? nullptr : prep;
    st = hip_status(launch_decode_partial(ln.sets, ln.n_sets, shape->head_dim, 1, ln.residual, s));
    if (st != RQ_OK) return st;
  }
  if (tail_len > 0) {
    // the tail: plain bf16 positions of every loop, one more split per row
    rq_shape ts = *shape;
    ts.seq_len = tail_len;
    const SplitPlan tp{1, (tail_len + kDecodeTile - 1) / kDecodeTile * kDecodeTile};
    DecodeArgs a{};
    fill_common(a, &ts, n_q_heads, q, softmax_scale, tp, workspace);
    a.rec_splits = rec_splits;
    a.split_base = prefix_recs;
    for (int i = 0; i < n_loops; ++i) {
      a.k[i] = tail_k[i];
      a.v[i] = tail_v[i];
    }
    a.loop_id[0] = 0;  // blockIdx.y selects the loop
    a.n_loops_launch = 1;
    a.n_rows = G;
    a.zero_residual = any_residual;
    st = hip_status(launch_decode_partial(&a, 1, shape->head_dim, n_loops, false, s));
    if (st != RQ_OK) return st;
  }
  return run_combine(shape, n_q_heads, n_loops, rec_splits, static_cast<const float*>(workspace), out,
                     any_residual, s, row_splits, balanced && tail_len > 0 ? prefix_recs : -1);
}

}  // namespace

extern "C" {

int rq_decode_attn(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                   const uint16_t* k_ref, const uint16_t* v_ref, const rq_loop_view* loops,
                   float softmax_scale, int32_t n_splits, float* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return decode_impl(shape, n_q_heads, n_loops, q, k_ref, v_ref, loops, nullptr, 0, nullptr, nullptr,
                     softmax_scale, n_splits, out, workspace, workspace_bytes, stream);
}

size_t rq_decode_attn_varlen_workspace(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops,
                                       int32_t n_splits, int32_t tail_len) {
  if (check_heads(shape, n_q_heads, n_loops) != RQ_OK || n_splits < 0 || tail_len < 0) return 0;
  if (n_splits == 0) return balanced_workspace_bytes(shape, n_q_heads, n_loops, tail_len);
  return workspace_bytes_for(shape, n_q_heads, n_loops,
                             plan_splits(shape, n_q_heads, n_loops, nullptr, n_splits).n_splits + (tail_len > 0 ? 1 : 0));
}

int rq_decode_attn_varlen(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                          const uint16_t* k_ref, const uint16_t* v_ref, const rq_loop_view* loops,
                          const int32_t* seq_lens, int32_t tail_len, const uint16_t* const* tail_k,
                          const uint16_t* const* tail_v, float softmax_scale, int32_t n_splits, float* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (seq_lens != nullptr && !aligned16(seq_lens)) return RQ_EALIGN;
  return decode_impl(shape, n_q_heads, n_loops, q, k_ref, v_ref, loops, seq_lens, tail_len, tail_k, tail_v,
                     softmax_scale, n_splits, out, workspace, workspace_bytes, stream);
}

int rq_decode_attn_paged(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                         const uint16_t* k_ref, const uint16_t* v_ref, const rq_loop_view* loops,
                         const rq_pages* pages, const int32_t* seq_lens, int32_t tail_len,
                         const uint16_t* const* tail_k, const uint16_t* const* tail_v, float softmax_scale,
                         int32_t n_splits, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (pages == nullptr) return RQ_EINVAL;
  if (seq_lens != nullptr && !aligned16(seq_lens)) return RQ_EALIGN;
  return decode_impl(shape, n_q_heads, n_loops, q, k_ref, v_ref, loops, seq_lens, tail_len, tail_k, tail_v,
                     softmax_scale, n_splits, out, workspace, workspace_bytes, stream, pages);
}

}  // extern "C"

namespace {

// Scratch of rq_decode_attn_noalloc: the decode workspace (split partials and
// rotated-query records) in a static device array, so that the call allocates
// nothing. Each GPU the library runs on holds its own copy until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory:
// its device address comes from hipGetSymbolAddress, taken once per device
// with that device current.
__device__ __align__(256) unsigned char scratch[RQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's address of `scratch`, or nullptr if it cannot be had.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  if (dev >= kMaxScratchDevices) {
    void* ptr = nullptr;
    return hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess ? ptr : nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int rq_decode_attn_noalloc(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                           const uint16_t* k_ref, const uint16_t* v_ref, const rq_loop_view* loops,
                           float softmax_scale, int32_t n_splits, float* out, void* stream) {
  // rq_decode_attn's checks first, without a workspace: they run on the host
  // and stop at the workspace check at the latest, before any HIP call
  const int st = decode_impl(shape, n_q_heads, n_loops, q, k_ref, v_ref, loops, nullptr, 0, nullptr, nullptr,
                             softmax_scale, n_splits, out, nullptr, 0, stream);
  if (st != RQ_EWORKSPACE) return st;
  if (rq_decode_attn_workspace(shape, n_q_heads, n_loops, n_splits) > (size_t)RQ_NOALLOC_SCRATCH_BYTES)
    return RQ_EWORKSPACE;
  void* ws = scratch_address();
  if (ws == nullptr) return RQ_EHIP;
  return decode_impl(shape, n_q_heads, n_loops, q, k_ref, v_ref, loops, nullptr, 0, nullptr, nullptr,
                     softmax_scale, n_splits, out, ws, (size_t)RQ_NOALLOC_SCRATCH_BYTES, stream);
}

int rq_decode_attn_bf16(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                        const uint16_t* const* k, const uint16_t* const* v, float softmax_scale,
                        int32_t n_splits, float* out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_heads(shape, n_q_heads, n_loops);
  if (st != RQ_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return RQ_EINVAL;
  if (n_splits < 0 || !isfinite(softmax_scale)) return RQ_EINVAL;
  for (int i = 0; i < n_loops; ++i) {
    if (k[i] == nullptr || v[i] == nullptr) return RQ_EINVAL;
  }
  if (!aligned16(q) || !aligned16(out)) return RQ_EALIGN;
  for (int i = 0; i < n_loops; ++i) {
    if (!aligned16(k[i]) || !aligned16(v[i])) return RQ_EALIGN;
  }
  const SplitPlan plan = plan_splits(shape, n_q_heads, n_loops, nullptr, n_splits);
  if (workspace == nullptr || workspace_bytes < workspace_bytes_for(shape, n_q_heads, n_loops, plan.n_splits))
    return RQ_EWORKSPACE;
  if (!aligned16(workspace)) return RQ_EALIGN;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = n_q_heads / shape->n_kv_heads;
  DecodeArgs a{};
  fill_common(a, shape, n_q_heads, q, softmax_scale, plan, workspace);
  for (int i = 0; i < n_loops; ++i) {
    a.k[i] = k[i];
    a.v[i] = v[i];
  }
  a.loop_id[0] = 0;  // blockIdx.y selects the loop
  a.n_loops_launch = 1;
  a.n_rows = G;
  st = hip_status(launch_decode_partial(&a, 1, shape->head_dim, n_loops, false, s));
  if (st != RQ_OK) return st;
  return run_combine(shape, n_q_heads, n_loops, plan.n_splits, static_cast<const float*>(workspace), out, false, s);
}

const char* rq_status_str(int status) {
  switch (status) {
    case RQ_OK: return "ok";
    case RQ_EINVAL: return "invalid argument";
    case RQ_EUNSUPPORTED: return "unsupported head_dim, bit width, head grouping or output type";
    case RQ_EALIGN: return "pointer not 16-byte aligned";
    case RQ_EWORKSPACE: return "workspace missing or too small";
    case RQ_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int32_t rq_format_version(void) { return RQ_FORMAT_VERSION; }

}  // extern "C"
