// Internal declarations shared by the librq HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq.h"

namespace rq {

constexpr int kMaxLoops = RQ_MAX_LOOPS;
constexpr int kGroup = RQ_GROUP;

// ---------------------------------------------------------------------------
// launch parameters
// ---------------------------------------------------------------------------

struct EncodeArgs {
  const uint16_t* x[kMaxLoops];
  uint32_t* codes[kMaxLoops];
  uint16_t* scales[kMaxLoops];
  int32_t bits[kMaxLoops];
  const uint16_t* ref;  // NULL: zero reference (rotation-only baseline)
  int32_t n_loops;
  int32_t refits;       // extra code / LS-scale alternations after the first fit
  // appending (pos != NULL): sources are [B][Hkv][t_new][D], outputs go to cache
  // position pos[b] + t of a [B][Hkv][s_cap] cache; ref_out receives the reference
  const int32_t* pos;
  int32_t t_new, n_kv_heads;
  int64_t s_cap;
  uint16_t* ref_out;
  // paged cache (block_table != NULL): outputs are [n_blocks][Hkv][2^log2_block][row]
  const int32_t* block_table;
  int32_t max_blocks, log2_block, n_blocks;
  int64_t n_vec;  // batch * n_kv_heads * seq_len
};

// One encode launch holds up to kMaxEncodeSets tensors of the same shape (K
// and V): blockIdx.y picks the tensor.
constexpr int kMaxEncodeSets = 2;
struct EncodeLaunch {
  EncodeArgs set[kMaxEncodeSets];
};

struct ReconstructArgs {
  const uint16_t* ref;  // NULL: zero reference (rotation-only baseline)
  const uint32_t* codes;
  const uint16_t* scales;
  void* out;
  int64_t n_vec;
};

// One decode launch covers `n_rows` query rows per (batch, kv head): rows
// r = li * G + j for slot li in [0, n_loops_launch) and j in [0, G). Row r
// reads the query of loop loop_id[li] + blockIdx.y, query head kvh * G + j.
// Slots are ordered INT8, INT4, INT3, INT2, reference-only. In the bf16
// baseline each launch has one slot (loop_id 0) and blockIdx.y picks the loop.
// One residual slot's tensors, together: a tile's issue loads all four with
// one scalar load.
struct SlotPtrs {
  const uint32_t* kc;
  const uint16_t* ks;
  const uint32_t* vc;
  const uint16_t* vs;
};

struct DecodeArgs {
  const uint16_t* q;                    // [n_loops_total][B][Hq][D]
  const uint16_t* k[kMaxLoops];         // per blockIdx.z: the K this block streams
  const uint16_t* v[kMaxLoops];
  int32_t bits[kMaxLoops];              // per slot li: 8, 4, 3, 2, then 0 (reference only)
  SlotPtrs slot[kMaxLoops];             // per slot li: its K / V codes and scales
  float* ws;                            // partials [n_loops_total][B][Hq][n_splits][2D + 2]
  const unsigned char* qprep;           // rotated-query records [n_loops_total][B][Hq], or NULL: a
                                        // residual launch at NB = 1 rotates the queries itself
  int32_t loop_id[kMaxLoops];           // per slot: the call's loop index of its rows (+ blockIdx.y)
  int32_t n8, n4, n3, n2;               // slot counts per width, in slot order; the rest bits 0
  int32_t n_loops_launch;               // slots (loops) whose rows this launch holds
  int32_t n_rows;                       // n_loops_launch * G
  int32_t group;                        // G = Hq / Hkv
  int32_t n_q_heads, n_kv_heads, batch, seq_len;
  int32_t n_splits, tokens_per_split;
  int32_t rec_splits, split_base;       // records per row in the workspace; this launch's first split
  const int32_t* seq_lens;              // device [B] prefix lengths, or NULL (all seq_len)
  // Length-balanced splits (balance_target > 0, seq_lens given): the launch
  // cuts the prefixes' 64-position units into splits of about equal length
  // whatever the prefix lengths, at most max_row_splits per (batch, kv head)
  // row and at most balance_target blocks (its grid) in all, and writes
  // sequence b's split count to row_splits[b] for the combine.
  int32_t balance_target, max_row_splits;
  int32_t* row_splits;
  // paged cache (block_table != NULL): tensors are [n_blocks][Hkv][2^log2_block][row];
  // position t of sequence b is in block block_table[b * max_blocks + (t >> log2_block)]
  const int32_t* block_table;
  int32_t max_blocks, log2_block, n_blocks;
  float scale_log2;                     // softmax scale * log2(e)
  int32_t lds_wave_bytes;               // per-wave LDS stride (set by the launcher)
  int32_t lds_res_base;                 // paired launches: this set's residual slots start after the
                                        // other set's (0 otherwise; set by the launcher)
  int32_t zero_residual;                // write a zero residual accumulator (reference-only launch)
};

// One partial launch holds up to kMaxSets argument sets over the same cache
// rows, each with its own query rows (at most 16 when there are two) and
// residual loops. With two, a block is a pair of waves, one per set, that
// share each tile's reference K and V through LDS, so the reference is read
// once for both sets.
constexpr int kMaxSets = 2;
struct DecodeLaunch {
  DecodeArgs set[kMaxSets];
  int32_t n_sets;
};

struct CombineArgs {
  const float* ws;
  float* out;
  int64_t n_out;       // n_loops * B * Hq
  int32_t n_splits;    // records per output row in the workspace
  int32_t residual;    // records carry a rotated-domain residual accumulator
  // Length-balanced splits: row_splits[b] (device) prefix records are valid
  // for sequence b, then the tail record at tail_slot (-1: none). NULL: all
  // n_splits records are valid.
  const int32_t* row_splits;
  int32_t batch, n_q_heads, tail_slot;
};

struct QueryPrepArgs {
  const uint16_t* q;            // [n_loops][B][Hq][D] bf16
  unsigned char* out;           // one record per query row
  int32_t bits[kMaxLoops];      // residual width of each loop (selects the offset constant)
  int64_t n_rows;               // n_loops * B * Hq
  int32_t batch, n_q_heads;
};

// ---------------------------------------------------------------------------
// launchers (defined in the .hip files); return hipGetLastError()
// ---------------------------------------------------------------------------

hipError_t launch_encode(const EncodeArgs* sets, int n_sets, int head_dim, hipStream_t stream);
hipError_t launch_reconstruct(const ReconstructArgs& a, int head_dim, int bits, int out_bf16, hipStream_t stream);
// sets[0 .. n_sets): argument sets of one launch (the same shape, splits,
// cache and paging; their own rows and loops)
hipError_t launch_decode_partial(const DecodeArgs* sets, int n_sets, int head_dim, int n_z, bool residual,
                                 hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_query_prep(const QueryPrepArgs& a, int head_dim, hipStream_t stream);

// bytes of one rotated-query record
int query_prep_bytes(int head_dim);

// tile of tokens one decode block iteration covers; split boundaries are multiples of it
constexpr int kDecodeTile = 64;

// blocks a decode launch aims at (enough to fill the chip twice over at two
// blocks per CU)
constexpr int kTargetBlocks = 512;

// Largest split count a length-balanced plan gives one (batch, kv head) row:
// twice the even share of kTargetBlocks, plus one, within the positions.
inline int balanced_max_row_splits(int64_t rows, int64_t seq_len) {
  const int64_t even = (kTargetBlocks + rows - 1) / rows;
  const int64_t units = (seq_len + kDecodeTile - 1) / kDecodeTile;
  const int64_t n = 2 * even + 1;
  return (int)(n < units ? n : (units < 1 ? 1 : units));
}
// Grid of a length-balanced launch, the most blocks its plan may use (the
// surplus ones exit): kTargetBlocks, so that all of it is resident at once
// (at least one block per row and kv head more than one per row), or every
// row at its cap.
inline int64_t balanced_max_blocks(int64_t rows, int64_t n_kv_heads, int64_t seq_len) {
  const int64_t spread = kTargetBlocks - rows > n_kv_heads ? kTargetBlocks - rows : n_kv_heads;
  const int64_t a = spread + rows, b = rows * balanced_max_row_splits(rows, seq_len);
  return a < b ? a : b;
}

// LDS one decode block may use (gfx950: 160 KB per workgroup)
constexpr int kMaxBlockLds = 160 * 1024;

// LDS bytes one decode wave stages per token tile for the given residual loops
int decode_wave_lds_bytes(int head_dim, const int32_t* bits, int n_loops);
// LDS bytes one residual loop of the given width adds to that (0 for bits 0)
int decode_loop_lds_bytes(int head_dim, int bits);

// LDS bytes one block of a partial launch takes (the largest over its sets);
// rotate: its residual blocks rotate the queries themselves (no prepared records)
int decode_launch_lds_bytes(const DecodeArgs* sets, int n_sets, int head_dim, bool residual, bool rotate);
// waves per block of a decode launch (2 for a paired launch, else 4 .. 8)
int decode_launch_waves(const DecodeArgs* sets, int n_sets, int head_dim, bool residual);

}  // namespace rq
