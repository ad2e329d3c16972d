/*
 * rq.h - C ABI of librq, the MI355X (gfx950) ResidualQuant hot path.
 *
 * ResidualQuant (newx.sg page, Abstract) stores the KV cache of a looped
 * Transformer like this: the final loop's K/V is kept as the reference, and
 * every earlier loop is kept only as a low-precision residual against it. The
 * residual is rotated and scaled by a least-squares fit. A loop-wise
 * mixed-precision table picks INT2 or INT4 per loop. The AI Summary on the
 * same page calls the mixed precision layer-wise instead; a table over
 * (layer, loop) with the further widths INT3 and INT8 covers both readings
 * (rq_encode_layers). The paperaft JSON page
 * (`summary`) adds that a serving stack must encode, decode and attend over
 * this custom format. This library provides exactly those operations:
 *
 *   rq_encode          rotate + quantize + pack the residuals of one tensor
 *   rq_encode_kv, rq_encode_append_kv, rq_encode_append_paged_kv  the same
 *                        for K and V together, in one launch
 *   rq_reconstruct     materialise one loop's K or V from ref + residual
 *   rq_decode_attn     fused reconstruct + single-query decode attention
 *   rq_decode_attn_bf16  the same decode attention over plain bf16 K/V per
 *                        loop (the uncompressed baseline)
 *   rq_encode_refit    rq_encode with extra code / LS-scale alternations
 *   rq_encode_append   encode new positions into a cache at per-sequence positions
 *   rq_decode_attn_varlen  decode over per-sequence prefix lengths plus a bf16 tail
 *   rq_encode_rotonly / rq_reconstruct_rotonly  the rotation-only baseline:
 *                        the same codec without a reference
 *   rq_encode_layers   rq_encode over several layers with a per-(layer, loop)
 *                        bit-width table
 *   rq_encode_append_paged / rq_decode_attn_paged  the serving step over a
 *                        block-paged cache
 *
 * FORMAT (RQ_FORMAT_VERSION 1)
 *   Dense tensors are [batch][n_kv_heads][seq_len][head_dim], head_dim
 *   contiguous. bf16 and fp16 travel as uint16_t bit patterns.
 *   Rotation: y = H r, where H is the normalised Sylvester Walsh-Hadamard
 *   matrix of order head_dim and r = x_loop - x_ref.
 *   Groups: 32 consecutive coordinates of y share one scale.
 *   Codes: one pass at the absmax step s0 = max|y_g| / (2^(b-1) - 1/2):
 *   c = clamp(floor(y / s0) + 2^(b-1), 0, 2^b - 1). The level is
 *   q = c - (2^(b-1) - 1/2), so INT2 levels are {-1.5, -0.5, 0.5, 1.5}.
 *   Widths: b in {2, 3, 4, 8}.
 *   Scale: s = <y_g, q_g> / <q_g, q_g>, stored as IEEE fp16 (round to nearest
 *   even, saturated at 65504). An all-zero group stores codes 2^(b-1) and
 *   s = 0, so a zero residual reconstructs the reference exactly.
 *   codes:  [batch][n_kv_heads][seq_len][head_dim*bits/32] uint32.
 *           b = 2, 4, 8: word w holds coordinates [(32/b)w, (32/b)(w+1));
 *           coordinate j of the word sits at bits [b*j, b*j+b).
 *           b = 3: two bit planes, so no code crosses a word. Words
 *           [0, head_dim/16) hold the low two bits of every code in the b = 2
 *           layout; words [head_dim/16, 3*head_dim/32) hold bit 2 of every
 *           code, coordinate j of word w at bit j.
 *   scales: [batch][n_kv_heads][seq_len][head_dim/32] fp16.
 *   Reconstruction: x_hat = x_ref + H (s * q).
 *
 * CONVENTIONS
 *   Every tensor pointer is a device pointer owned by the caller, and must be
 *   16-byte aligned. The library allocates nothing and keeps no pointer after
 *   a call returns. Kernels are enqueued on `stream` (a hipStream_t; NULL
 *   means the default stream) and the library never synchronises. Inputs must
 *   stay valid until the stream has run the work. Outputs must not alias
 *   inputs. The library holds no state, so calls on different streams may run
 *   concurrently.
 *   Every call returns an rq_status. All checks except RQ_EHIP run on the host
 *   before any HIP call, and a failed check enqueues nothing. RQ_EHIP reports
 *   a launch error; faults inside a kernel show up at the caller's next
 *   synchronisation.
 */
#ifndef RQ_H
#define RQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RQ_FORMAT_VERSION 1
#define RQ_GROUP 32
#define RQ_MAX_LOOPS 8
#define RQ_MAX_REFITS 16
#define RQ_MAX_LAYERS 4096
#define RQ_NOALLOC_SCRATCH_BYTES (32u << 20) /* device scratch of rq_decode_attn_noalloc */

typedef enum rq_status {
  RQ_OK = 0,
  RQ_EINVAL = -1,        /* null pointer, non-positive size, n_q_heads % n_kv_heads != 0,
                            n_loops outside [1, RQ_MAX_LOOPS], non-finite softmax scale */
  RQ_EUNSUPPORTED = -2,  /* head_dim not in {64, 128}, bits not in {0, 2, 3, 4, 8} (not 0
                            for the encoders), query heads per kv head above 32, bad out_dtype,
                            decode with seq_len * head_dim * 2 above 2^31 - 1 bytes */
  RQ_EALIGN = -3,        /* a pointer is not 16-byte aligned */
  RQ_EWORKSPACE = -4,    /* workspace NULL or smaller than the size query returned */
  RQ_EHIP = -5           /* the HIP runtime reported an error at launch */
} rq_status;

enum { RQ_OUT_F32 = 0, RQ_OUT_BF16 = 1 };

typedef struct rq_shape {
  int32_t batch;
  int32_t n_kv_heads;
  int32_t seq_len;
  int32_t head_dim; /* 64 or 128 */
} rq_shape;

/* A block-paged cache (the serving-step calls *_paged). Every paged tensor is
   [n_blocks][n_kv_heads][block_size][row] (row: head_dim bf16 for the
   reference, head_dim*bits/32 words for codes, head_dim/32 fp16 for scales),
   and position t of sequence b lives in block block_table[b * max_blocks +
   t / block_size] at offset t % block_size. Blocks may be shared or in any
   order; a table entry outside [0, n_blocks) marks a block that is not there:
   its positions take no attention weight and appends to it write nothing. */
typedef struct rq_pages {
  const int32_t* block_table; /* device int32 [batch][max_blocks] */
  int32_t max_blocks;         /* table entries per sequence */
  int32_t block_size;         /* positions per block: a power of two, at least 64 */
  int32_t n_blocks;           /* blocks in every paged tensor */
} rq_pages;

/* One loop of the cache as rq_decode_attn reads it. bits = 0 marks the final
   loop (the reference itself; code and scale pointers are ignored and may be
   NULL). bits = 2, 3, 4 or 8 is a residual loop in the format above. */
typedef struct rq_loop_view {
  int32_t bits;
  const uint32_t* k_codes;
  const uint16_t* k_scales;
  const uint32_t* v_codes;
  const uint16_t* v_scales;
} rq_loop_view;

/* Encode the residuals of n_loops loops of one tensor (K or V) against the
 * final-loop reference (ResidualQuant, newx.sg page, Abstract: the earlier
 * loops are stored as rotated, least-squares-scaled low-bit residuals).
 * The reference is read once for all loops.
 *   x[i]      bf16 [B][Hkv][S][D], loop i's states (host array of n_loops device pointers)
 *   bits[i]   2, 3, 4 or 8 (host array)
 *   ref       bf16 [B][Hkv][S][D], the final loop
 *   codes[i]  out: uint32 [B][Hkv][S][D*bits[i]/32]
 *   scales[i] out: fp16  [B][Hkv][S][D/32]
 * The inputs must be finite. The output is deterministic: it depends only on
 * the inputs. */
int rq_encode(const rq_shape* shape, int32_t n_loops, const uint16_t* const* x, const int32_t* bits,
              const uint16_t* ref, uint32_t* const* codes, uint16_t* const* scales, void* stream);

/* rq_encode of K and V together, in one launch: the same as rq_encode(kx,
 * k_ref, k_codes, k_scales) followed by rq_encode(vx, v_ref, v_codes,
 * v_scales) with the same bits, and bit-identical to it. A layer's K and V
 * share the loop table; one launch saves the second launch's ramp and the
 * first one's tail. Arguments as in rq_encode, once per tensor; the checks are
 * those of two rq_encode calls and nothing is enqueued if either fails.
 */
int rq_encode_kv(const rq_shape* shape, int32_t n_loops, const uint16_t* const* kx, const uint16_t* const* vx,
                 const int32_t* bits, const uint16_t* k_ref, const uint16_t* v_ref, uint32_t* const* k_codes,
                 uint16_t* const* k_scales, uint32_t* const* v_codes, uint16_t* const* v_scales, void* stream);

/* rq_encode with `refits` extra alternations of the two least-squares
 * half-steps after the first fit (ResidualQuant, newx.sg page, AI Summary:
 * the scale is a least-squares fit; the alternation applies that fit in turn
 * to the codes). Each round first reassigns every code to the nearest level
 * at the current scale s: c = clamp(floor(y / s) + 2^(b-1), 0, 2^b - 1).
 * Then it refits s = <y, q> / <q, q>. Neither step can raise |y - s q|.
 * refits = 0 is rq_encode. The format is unchanged, so rq_reconstruct and
 * rq_decode_attn read the output as they read rq_encode's.
 *   refits  0 .. RQ_MAX_REFITS (RQ_EINVAL otherwise); other arguments as rq_encode. */
int rq_encode_refit(const rq_shape* shape, int32_t n_loops, const uint16_t* const* x, const int32_t* bits,
                    const uint16_t* ref, uint32_t* const* codes, uint16_t* const* scales, int32_t refits,
                    void* stream);

/* Append t_new new positions per sequence to a residual cache: the serving
 * step around the hot path (ResidualQuant, paperaft JSON page, `summary`: the
 * cache lives in this custom format inside a serving stack). A position's
 * earlier loops can only be encoded once its final loop exists. This call
 * encodes the new positions' loops against their final-loop states, writes
 * the codes and scales at each sequence's write position, and copies the
 * final-loop states into the bf16 reference cache.
 *   cache      shape of the cache tensors; cache->seq_len is their capacity S_cap
 *   x[i]       bf16 [B][Hkv][t_new][D]: loop i of the new positions (host array)
 *   bits[i]    2, 3, 4 or 8 (host array)
 *   ref_new    bf16 [B][Hkv][t_new][D]: the final loop of the new positions
 *   pos        device int32 [B]: sequence b's new positions go to pos[b] + t,
 *              t < t_new; a position outside [0, S_cap) is skipped (not written)
 *   ref_cache  bf16 [B][Hkv][S_cap][D]: receives ref_new at those positions
 *   codes[i], scales[i]  the cache's [B][Hkv][S_cap][...] code and scale tensors
 * Codes and scales are those rq_encode gives for the same vectors. */
int rq_encode_append(const rq_shape* cache, int32_t n_loops, int32_t t_new, const uint16_t* const* x,
                     const int32_t* bits, const uint16_t* ref_new, const int32_t* pos, uint16_t* ref_cache,
                     uint32_t* const* codes, uint16_t* const* scales, void* stream);

/* rq_encode_append into a block-paged cache (rq_pages).
 *   cache      batch, n_kv_heads and head_dim of the cache; cache->seq_len is
 *              the capacity of one sequence, pages->max_blocks * pages->block_size
 *              (RQ_EINVAL otherwise)
 *   ref_pages  bf16 [n_blocks][Hkv][block_size][D]: receives ref_new
 *   codes[i], scales[i]  paged tensors [n_blocks][Hkv][block_size][...]
 *   block_size not a power of two of at least 64: RQ_EUNSUPPORTED.
 * A position outside [0, capacity), or in a block whose table entry is not
 * valid, is skipped. Other arguments and the output values as rq_encode_append;
 * with t_new = S and pos = 0 this is the encode of a whole prefill into pages. */
int rq_encode_append_paged(const rq_shape* cache, const rq_pages* pages, int32_t n_loops, int32_t t_new,
                           const uint16_t* const* x, const int32_t* bits, const uint16_t* ref_new,
                           const int32_t* pos, uint16_t* ref_pages, uint32_t* const* codes,
                           uint16_t* const* scales, void* stream);

/* rq_encode_append of K and V together, in one launch (bit-identical to the
 * two calls with the same pos and bits). A serving step appends both tensors
 * of every layer; these launches are small enough that the second launch's
 * latency is most of its cost. Arguments as in rq_encode_append, once per
 * tensor.
 */
int rq_encode_append_kv(const rq_shape* cache, int32_t n_loops, int32_t t_new, const uint16_t* const* kx,
                        const uint16_t* const* vx, const int32_t* bits, const uint16_t* k_ref_new,
                        const uint16_t* v_ref_new, const int32_t* pos, uint16_t* k_ref_cache, uint16_t* v_ref_cache,
                        uint32_t* const* k_codes, uint16_t* const* k_scales, uint32_t* const* v_codes,
                        uint16_t* const* v_scales, void* stream);

/* rq_encode_append_paged of K and V together, in one launch (bit-identical to
 * the two calls). Arguments as in rq_encode_append_paged, once per tensor.
 */
int rq_encode_append_paged_kv(const rq_shape* cache, const rq_pages* pages, int32_t n_loops, int32_t t_new,
                              const uint16_t* const* kx, const uint16_t* const* vx, const int32_t* bits,
                              const uint16_t* k_ref_new, const uint16_t* v_ref_new, const int32_t* pos,
                              uint16_t* k_ref_pages, uint16_t* v_ref_pages, uint32_t* const* k_codes,
                              uint16_t* const* k_scales, uint32_t* const* v_codes, uint16_t* const* v_scales,
                              void* stream);

/* Materialise one loop: out = ref + H (s * q) (ResidualQuant, newx.sg page,
 * Abstract: the residual format keeps reconstruction cheap).
 *   bits 0 copies ref. out_dtype RQ_OUT_F32 writes float [B][Hkv][S][D];
 *   RQ_OUT_BF16 writes bf16 bits rounded to nearest even. */
int rq_reconstruct(const rq_shape* shape, int32_t bits, const uint16_t* ref, const uint32_t* codes,
                   const uint16_t* scales, int32_t out_dtype, void* out, void* stream);

/* Rotation-only baseline: the same codec with a zero reference. Each of
 * n_states states (every loop, the final one included) is rotated and
 * quantized directly, with no bf16 reference kept. This is the comparison
 * point the ResidualQuant page names (newx.sg page, Abstract: the residuals
 * are set against a rotation-based baseline at the same bit widths).
 *   x[i]      bf16 [B][Hkv][S][D] (host array of n_states device pointers)
 *   bits[i]   2, 3, 4 or 8 (host array)
 *   codes[i], scales[i]  out, as in rq_encode
 * Codes and scales are those rq_encode gives for the same states against an
 * all-zero reference. Errors as rq_encode. */
int rq_encode_rotonly(const rq_shape* shape, int32_t n_states, const uint16_t* const* x, const int32_t* bits,
                      uint32_t* const* codes, uint16_t* const* scales, void* stream);

/* Materialise one rotation-only state: out = H (s * q), the output of
 * rq_reconstruct with an all-zero reference. bits must be 2, 3, 4 or 8
 * (RQ_EUNSUPPORTED otherwise); output types as rq_reconstruct. */
int rq_reconstruct_rotonly(const rq_shape* shape, int32_t bits, const uint32_t* codes, const uint16_t* scales,
                           int32_t out_dtype, void* out, void* stream);

/* Encode the residual caches of n_layers layers with a per-(layer, loop)
 * bit-width table (ResidualQuant, newx.sg page: the Abstract calls the mixed
 * precision loop-wise, the AI Summary layer-wise; a table over both holds
 * either). Each layer has its own final-loop reference and n_loops earlier
 * loops; the call is n_layers rq_encode calls on the stream, with every
 * argument of every layer checked before the first launch. Decoding a layer
 * takes that layer's row of the table as its loops' bits.
 *   n_layers     1 .. RQ_MAX_LAYERS
 *   x            host array [n_layers * n_loops] of device pointers, layer-major:
 *                x[l * n_loops + i] is loop i of layer l, bf16 [B][Hkv][S][D]
 *   bits_table   host array [n_layers * n_loops]: 2, 3, 4 or 8
 *   ref          host array [n_layers]: layer l's final loop, bf16 [B][Hkv][S][D]
 *   codes, scales  host arrays [n_layers * n_loops] of outputs, as in rq_encode
 * All layers share `shape`. Errors as rq_encode. */
int rq_encode_layers(const rq_shape* shape, int32_t n_layers, int32_t n_loops, const uint16_t* const* x,
                     const int32_t* bits_table, const uint16_t* const* ref, uint32_t* const* codes,
                     uint16_t* const* scales, void* stream);

/* Split count rq_decode_attn / rq_decode_attn_bf16 will use for a request of
 * n_splits (0 = automatic). Splits hold whole 64-position units. The automatic
 * count depends on the shape, n_q_heads, n_loops and the loops' widths: it is
 * the one with the least modelled time ceil(B*Hkv*n / R) * (1/n + 384/seq_len),
 * R being the partial blocks the device holds at once (512 for at most 16
 * query rows per kv head, 256 when those rows' loops stage too much per tile
 * for two blocks per CU (INT8 loops, or several INT4 loops), 1024 for more
 * rows of at most 16 heads each, 256 above 16 heads).
 *   bits: host array [n_loops] of the call's widths (0, 2, 3, 4 or 8, as in
 *         its rq_loop_view array), or NULL for widths that fit two blocks per
 *         CU; rq_decode_attn_bf16 plans as if NULL.
 * Host only. Returns <= 0 on invalid arguments. */
int32_t rq_decode_attn_splits(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const int32_t* bits,
                              int32_t n_splits);

/* Workspace bytes needed by rq_decode_attn and rq_decode_attn_bf16 for these
 * arguments, whatever the loops' widths (an automatic count sizes for the
 * larger of its two possible plans). Host only; 0 on invalid arguments. The
 * caller allocates it. */
size_t rq_decode_attn_workspace(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, int32_t n_splits);

/* Fused decode attention over the residual cache (ResidualQuant, newx.sg
 * page, Abstract: a smaller cache means less KV memory traffic per decode
 * step). For each loop i, batch b and query head h, with kv = h / (Hq/Hkv):
 *   k_hat_t = k_ref_t + H (s_k * q_k)_t   (k_ref_t alone when bits = 0)
 *   v_hat_t likewise,
 *   out[i][b][h] = sum_t softmax_t(scale * q[i][b][h] . k_hat_t) v_hat_t
 * over all seq_len cached positions, with no mask. The reference is streamed
 * once for all loops of the call.
 *   q        bf16 [n_loops][B][Hq][D]
 *   k_ref, v_ref  bf16 [B][Hkv][S][D]
 *   loops    host array [n_loops]
 *   out      float [n_loops][B][Hq][D]
 *   softmax_scale: usually 1/sqrt(D); n_splits: 0 = automatic.
 * Results are identical from run to run for the same n_splits.
 *
 * Numeric envelope. Scores, the softmax and every sum are fp32. The
 * reference products take the stored bf16 values as they are (exact
 * products). The rotated query Hq enters the residual scores as an fp16
 * pair hi + lo (about 2^-22 relative). Softmax weights enter the reference
 * PV as a bf16 pair hi + lo (about 2^-16 relative) and the residual PV as
 * fp16 weights P * s, each rounded once to nearest (2^-11 relative). The
 * last is the leading term: a row's error is at most about
 * 2^-11 * max_t |v_hat_t - v_ref_t| / max|out| before averaging over
 * tokens, so residuals up to a few times the output's magnitude stay within
 * a row error (max_i |out - out*| / max_i |out*|) of 2e-3 against fp64.
 * Tested there: encoder outputs whose residual is as large as the reference
 * at widths 2, 3, 4 and 8, Gaussian and with heavy tails (channels x20,
 * Student-t(4) values), at 4, 16 and 20 query heads per KV head; and the
 * encoder's own outputs at 8K and 32K positions.
 * Outside it: rotated query coordinates beyond the fp16 range (|Hq| >
 * 65504), non-finite inputs, and residuals far larger than the reference. */
int rq_decode_attn(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                   const uint16_t* k_ref, const uint16_t* v_ref, const rq_loop_view* loops,
                   float softmax_scale, int32_t n_splits, float* out, void* workspace,
                   size_t workspace_bytes, void* stream);

/* rq_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same computation and kernels, with the same results (bit-identical for
 * the same n_splits), but no workspace argument: the split partials and the
 * rotated-query records go to a static device array of
 * RQ_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it
 * runs on until the process ends. The call allocates nothing and calls no
 * allocating routine; it takes the array's device address once per device
 * (hipGetSymbolAddress) with that device current.
 *   Arguments, checks and errors as rq_decode_attn; in addition
 *   RQ_EWORKSPACE when rq_decode_attn_workspace for these arguments exceeds
 *   RQ_NOALLOC_SCRATCH_BYTES (nothing is enqueued), and RQ_EHIP if the
 *   array's address cannot be had.
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents (no part of it needs to start at zero: every value a call
 * reads back, the same call wrote first). Calls on one GPU whose kernels
 * overlap (different streams, or different host threads) race on the array
 * and give undefined results: serialise them, or use rq_decode_attn with a
 * workspace per stream. */
int rq_decode_attn_noalloc(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                           const uint16_t* k_ref, const uint16_t* v_ref, const rq_loop_view* loops,
                           float softmax_scale, int32_t n_splits, float* out, void* stream);

/* Decode attention over a partly filled residual cache, plus the positions
 * not yet encoded: the serving-loop form of rq_decode_attn (paperaft JSON
 * page, `summary`: decoding from the custom format in a serving stack).
 * Sequence b attends to its first seq_lens[b] cached positions and then to
 * tail_len positions per loop kept in bf16. In a looped model these are the
 * current position's states of each loop, which can only be encoded once its
 * final loop has run.
 *   shape      the cache tensors; shape->seq_len is their capacity S_cap
 *   seq_lens   device int32 [B], each in [0, S_cap] (values outside are clamped);
 *              NULL means S_cap for every sequence
 *   tail_len   0 (no tail) or the number of bf16 tail positions per sequence
 *   tail_k[i], tail_v[i]  bf16 [B][Hkv][tail_len][D] for loop i (host arrays of
 *              device pointers; ignored when tail_len = 0)
 * A row with no position at all (seq_lens[b] = 0 and no tail) is all zeros.
 * With seq_lens given and n_splits = 0 the splits follow the actual lengths:
 * each sequence's prefix is cut into equal splits, sized so that every block
 * of the launch streams about the same number of positions (at most
 * 2 * ceil(512 / (B * Hkv)) + 1 splits per sequence). An explicit n_splits
 * cuts the capacity S_cap instead, as rq_decode_attn does. Results are
 * identical from run to run for the same lengths and n_splits.
 * Other arguments, the output and the errors are as in rq_decode_attn. The
 * workspace size comes from rq_decode_attn_varlen_workspace (n_splits = 0:
 * room for the length-following plan, whatever the lengths). */
size_t rq_decode_attn_varlen_workspace(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops,
                                       int32_t n_splits, int32_t tail_len);
int rq_decode_attn_varlen(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                          const uint16_t* k_ref, const uint16_t* v_ref, const rq_loop_view* loops,
                          const int32_t* seq_lens, int32_t tail_len, const uint16_t* const* tail_k,
                          const uint16_t* const* tail_v, float softmax_scale, int32_t n_splits, float* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* rq_decode_attn_varlen over a block-paged cache (rq_pages): k_ref, v_ref and
 * every loop view's code and scale tensors are paged tensors
 * [n_blocks][Hkv][block_size][...]; the tail tensors stay dense
 * [B][Hkv][tail_len][D]. shape->seq_len is the capacity of one sequence,
 * pages->max_blocks * pages->block_size (RQ_EINVAL otherwise); block_size not a
 * power of two of at least 64 is RQ_EUNSUPPORTED. The workspace size comes
 * from rq_decode_attn_varlen_workspace with the same shape. The result is that
 * of rq_decode_attn_varlen over the cache the table describes. */
int rq_decode_attn_paged(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                         const uint16_t* k_ref, const uint16_t* v_ref, const rq_loop_view* loops,
                         const rq_pages* pages, const int32_t* seq_lens, int32_t tail_len,
                         const uint16_t* const* tail_k, const uint16_t* const* tail_v, float softmax_scale,
                         int32_t n_splits, float* out, void* workspace, size_t workspace_bytes, void* stream);

/* The uncompressed baseline: the same decode attention where loop i attends
 * over its own bf16 K/V, k[i] and v[i] (host arrays of device pointers, each
 * bf16 [B][Hkv][S][D]). ResidualQuant (newx.sg page, Abstract) measures its
 * decode throughput against a BF16 KV cache; this is that cache, decoded by
 * the same kernels without residual loops, so the two differ only in the
 * bytes they stream. Same q / out layout, workspace query and split rule;
 * errors as rq_decode_attn. */
int rq_decode_attn_bf16(const rq_shape* shape, int32_t n_q_heads, int32_t n_loops, const uint16_t* q,
                        const uint16_t* const* k, const uint16_t* const* v, float softmax_scale,
                        int32_t n_splits, float* out, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Static description of a status code. */
const char* rq_status_str(int status);

/* RQ_FORMAT_VERSION of the library as built. */
int32_t rq_format_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H */
